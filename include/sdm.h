/*
 * sdm.h - C ABI of the MI355X (gfx950) forward hot path of the chunked sparse-delta-memory
 * (SDM) recurrence: Phase 1 (the memory-independent per-chunk quantities) and the DW
 * decay-and-write step; beside them the read side of a step and the backward movers (GDS, GWR,
 * PA).
 *
 * Conventions shared by every entry point
 *  - All array arguments are DEVICE pointers owned by the caller. The library allocates no
 *    memory, keeps no pointer after returning and never synchronizes: work is enqueued on the
 *    caller's stream `st` (hipStream_t; 0 = the null stream).
 *  - The shape and argument checks, and the once-per-device set-up (the device's LDS limit, the
 *    kernels' dynamic-LDS attributes), run on the host before anything is enqueued. Any non-zero
 *    status from a check or the set-up means nothing was launched; sdm_last_error() then returns
 *    a message naming the failed check (thread-local, valid until the next call on that thread).
 *    An entry point that enqueues several kernels makes no other runtime call between them, so
 *    the only later failure is a launch the runtime itself rejects (SDM_EHIP), which the checks
 *    rule out for shapes they accept.
 *  - Device code never traps on inputs that pass the checks. Slot ids outside the ranges
 *    stated below are the caller's contract (results are unspecified, memory stays in bounds
 *    for Phase 1; DW writes the rows the records name).
 *  - Outputs are bitwise reproducible run to run for fixed inputs and shapes: sorts are
 *    stable, scans combine in a fixed tree, every output element has one writer, and no
 *    floating-point atomics are used.
 *
 * Notation (page "sparse_delta_memory/cuda/phase1_cuda.py", module docstring and the Outputs /
 * Records comments): a chunk c holds C tokens; token t writes W slots (K entries, lanes 0..W-1)
 * and reads R slots (Q entries). Entry r = t (W + R) + j of a chunk is K lane j when j < W and
 * Q lane j - W otherwise. Chunk c is step c / P of stream c % P; stream p's local slot of an
 * absolute id is id - p * stream_offset. Tokens t >= valid_last of chunks c >= first_partial
 * are invalid (masked): their entries are sorted after all valid entries, in entry order, each
 * as a group of its own, and their values / gates / token rows are never read.
 */
#ifndef SDM_H
#define SDM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sdm_status {
    SDM_OK = 0,
    SDM_EINVAL = -1,       /* a required pointer is NULL, or an argument is out of range */
    SDM_ESHAPE = -2,       /* shape outside the supported ranges (C, W, R, row length, ti) */
    SDM_EALIGN = -3,       /* a pointer is not aligned as required */
    SDM_EUNSUPPORTED = -4, /* a valid shape this build does not implement */
    SDM_EWORKSPACE = -5,   /* workspace missing or smaller than sdm_phase1_workspace() */
    SDM_EHIP = -6          /* a HIP launch or attribute call failed */
} sdm_status;

typedef enum sdm_dtype {
    SDM_F32 = 0,
    SDM_BF16 = 1
} sdm_dtype;

/* Shape of one Phase-1 call over N chunks. */
typedef struct sdm_p1_shape {
    int32_t N;              /* chunks, >= 0 */
    int32_t C;              /* tokens per chunk, 1..256 */
    int32_t W;              /* K entries per token, 1..256 */
    int32_t R;              /* Q entries per token, 1..256 */
    int32_t P;              /* independent streams, >= 1 */
    int32_t key_bits;       /* every valid local slot is < 2^key_bits; 1..30 */
    int64_t stream_offset;  /* slot offset between streams (>= 0) */
    int32_t first_partial;  /* chunks c >= first_partial are ragged (0..N; N: none) */
    int32_t valid_last;     /* valid tokens of a ragged chunk, 0..C */
    int32_t tile_len;       /* L of the tile bounds tiles_k, >= 1 */
    int32_t g_lane_stride;  /* layout of the gates g: 0 = one gate per token, [N, C]; 1 = one gate per
                               (token, K lane), [N, C, W] (page "sparse_delta_memory/cuda/phase1_cuda.py",
                               p1_scan_kernel: the gate is read at token * width + lane * stride). With 1,
                               a token that writes one slot from several lanes applies the gate of the
                               lowest of those lanes (its other writes there are repeats). */
    int32_t idx_bytes;      /* width of the slot ids k_idx / q_idx: 0 or 4 = int32, 8 = int64 (every
                               absolute slot is below 2^31 either way) */
    int32_t val_bytes;      /* type of the values k_val / q_val and of the value-typed outputs cpe,
                               k_eff, q_w: 0 or 4 = float32, 2 = bfloat16 (page
                               "sparse_delta_memory/cuda/phase1_cuda.py": the value type of the Outputs
                               struct). With bfloat16, each of those outputs is its float32 result
                               rounded to bfloat16 (nearest even), krec's cpe field holds that rounded
                               cpe widened to float32 (so sdm_dw_step scales by it), and every other
                               output is computed from the values widened exactly to float32. */
    int32_t tiled;          /* 0: rows of up to 16384 entries are sorted and scanned on chip by one
                               workgroup per chunk, longer rows (up to 2^17 entries) take the tiled
                               path; 1: every row takes the tiled path. The tiled path (page
                               "sparse_delta_memory/cuda/phase1_cuda.py": the merge rounds of rows too
                               long for one on-chip sort) works from global memory in tiles of 16384
                               entries: a stable radix sort through two workspace buffers, then the
                               reverse and forward scans tile by tile with carries. Its integer outputs
                               equal the on-chip path's bit for bit; its float outputs meet the same
                               tolerance. */
    int32_t lds_budget;     /* LDS bytes per workgroup the on-chip sort/scan kernel plans with: 0 = the
                               whole 160 KB; a smaller value (16384 .. 163840) makes it take narrower radix
                               digits, stage fewer values in LDS and write its outputs in more sweeps, with
                               every output bit for bit the same (a test knob for those paths). A budget
                               the shape cannot fit in is refused with SDM_EUNSUPPORTED. The tiled path
                               and the pair kernel ignore it. */
    int32_t pair_walk;      /* 0: slot groups with at least 16 valid K entries are summed as a dense
                               contraction when LDS allows (page "sparse_delta_memory/cuda/phase1_cuda.py",
                               p1_pairs_hc_kernel: the hot/cold form); 1: every group is walked in the
                               ordered form. A and QK of the two forms agree within the float32 bound,
                               not bit for bit; every other output is the same. */
} sdm_p1_shape;

/*
 * Phase-1 buffers. Entry-order fields are [N, C, W] (K) or [N, C, R] (Q), row-major.
 * Sorted-kind fields follow the chunk's sorted order restricted to one kind ("K-only row",
 * length C*W; "Q-only row", length C*R), padding (invalid) entries included.
 * A NULL output pointer skips that output, except spay_k, krec and tiles_k, which the DW step
 * consumes and which are always required.
 */
typedef struct sdm_p1_io {
    /* inputs */
    const void* k_idx;      /* [N, C, W] absolute slot ids of the writes, int32 or int64 (idx_bytes) */
    const void* q_idx;      /* [N, C, R] absolute slot ids of the reads, same type */
    const void* k_val;      /* [N, C, W] write values, float32 or bfloat16 (val_bytes) */
    const void* q_val;      /* [N, C, R] read values, same type */
    const float* g;         /* gates (log decays): [N, C] per token, or [N, C, W] per (token, K lane)
                               when g_lane_stride = 1 */
    /* entry-order outputs */
    float* log_k;           /* [N, C, W] log-cumsum of the slot's gates up to and including the entry */
    float* rex;             /* [N, C, W] sum of the slot's later gates in the chunk */
    void* cpe;              /* [N, C, W] exp(total gate of the slot in the chunk); value type */
    void* k_eff;            /* [N, C, W] k_val * exp(log_k); value type */
    int8_t* is_last;        /* [N, C, W] last valid K entry of its slot */
    int8_t* is_only;        /* [N, C, W] only valid K entry of its slot */
    int32_t* pos_k;         /* [N, C, W] sorted position | min(after,127)<<17 | min(peers,127)<<24 */
    float* log_q;           /* [N, C, R] log-cumsum seen by the read (its own token's writes included) */
    void* q_w;              /* [N, C, R] q_val * exp(log_q); value type */
    int32_t* pos_q;         /* [N, C, R] as pos_k, peers counted among valid Q entries */
    int8_t* q_last;         /* [N, C, R] last valid Q entry of its slot */
    int8_t* q_only;         /* [N, C, R] only valid Q entry of its slot */
    /* sorted-kind outputs */
    int32_t* spay_k;        /* [N, C*W] K-only row elements: entry bits 0-17 (lane 0-7, Q bit 8, token
                               9-16, invalid 17), distance to the kind's first entry of the group in
                               bits 18-29 (saturating at 4095), LAST bit 30, FIRST bit 31; padding is
                               FIRST|LAST. REQUIRED. */
    int32_t* spay_q;        /* [N, C*R] Q-only row elements, same layout */
    int32_t* krec;          /* [N, C*W, 4] {spay_k element, absolute slot, f32 bits of k*exp(rex),
                               f32 bits of cpe}; padding {element, 0, +0, 1.0f}. 16-byte aligned.
                               REQUIRED. */
    int32_t* tiles_k;       /* [N, ceil(C*W/L) + 1]: first index >= t*L of the K-only row holding a
                               FIRST (C*W if none), then C*W. REQUIRED. */
    float* a;               /* [N, C, C] A[i,j] (j < i), zeros elsewhere */
    float* qk;              /* [N, C, C] QK[i,j] (j <= i), zeros elsewhere */
    int32_t* repeats;       /* [N] per chunk: K entries whose group predecessor is a K entry of the
                               same token (their gate is not applied again) */
    int32_t* perm;          /* [N, C*(W+R)] the chunk's sorted order: entry index r = t*(W+R) + j at
                               each sorted position (the permutation the stable sort by slot makes;
                               invalid entries last, in entry order) */
    void* workspace;        /* device scratch, 16-byte aligned, >= sdm_phase1_workspace(shape) */
    size_t workspace_bytes;
    hipEvent_t* events;     /* optional (NULL: none): 4 caller-created events bound to the kernels'
                               own start and end (hipExtLaunchKernel): [0], [1] the sort/scan kernel,
                               [2], [3] the pair kernel (an event of a kernel that is not launched,
                               such as the pair kernel when a and qk are both NULL, is not recorded) */
    int32_t* status;        /* debug, optional (NULL: off): when set, the sort/scan kernel checks every
                               valid entry's slot id (local slot in [0, 2^key_bits), id >= 0) and sets bit
                               0 of *status (an atomic OR) if one is out of range. The caller zeroes the
                               word before the call and reads it once the stream has run the call (a
                               device-side error cannot be a return code: nothing here synchronizes).
                               Out-of-range ids only reach the sort as masked keys, so Phase 1 stays in
                               bounds; the records they leave must not be given to sdm_dw_step. */
    int32_t* gord_k;        /* optional [N, C*W] (NULL: skipped): per K-only-row position, the dense ordinal of
                               its group among the chunk's groups with a valid write, in K-row (slot) order;
                               -1 for padding. It is the row index of the dense compact snapshot (page
                               "sparse_delta_memory/cuda/mover_fx_cuda.py", module docstring: a group's row
                               at its dense ordinal in the chunk). Written by a small scan kernel on st. */
    int32_t defer_pairs;    /* 0: the pair sums (a, qk) are computed by this call. 1: this call leaves
                               them for sdm_phase1_pairs (the sort/scan kernel still writes their inputs
                               into the workspace), so that a caller can run them on another stream
                               beside work that needs only the other outputs (DW needs krec alone). */
} sdm_p1_io;

/*
 * Device workspace bytes one sdm_phase1 call needs (sorted-order pair records and the inverse
 * permutation of every chunk). Returns 0 for a shape sdm_phase1 would refuse.
 */
size_t sdm_phase1_workspace(const sdm_p1_shape* shape);

/*
 * Phase 1 of N chunks (page "sparse_delta_memory/cuda/phase1_cuda.py": module docstring for the
 * quantities; p1_keys_zw_kernel for keys and payloads; p1_scan_kernel for groups, repeats, packed
 * positions, kind rows, records and tile bounds; p1_pairs_kernel's comment for A and QK).
 *
 * Per chunk: entries are sorted stably by local slot (invalid entries last, in entry order); a
 * group is a run of valid entries with one slot. A valid K entry contributes its token's gate g,
 * except a repeat (its group predecessor is a K entry of the same token), which contributes 0.
 * log_k / log_q are the inclusive per-group cumsums of these contributions, rex the sum after the
 * entry, cpe = exp(group total). A[i,j] sums k_e k_f exp(log_k_e - log_k_f) over K entries e of
 * token i and earlier K entries f of token j != i in the same group; QK[i,j] sums
 * q_e k_f exp(log_q_e - log_k_f) over Q entries e of token i and earlier K entries f of token j.
 * Invalid entries: log 0, rex 0, cpe 1, k_eff / q_w 0, flags 0, pos = sorted position.
 *
 * Requirements: C*(W+R) <= 2^17 (rows past 16384 entries take the tiled path); 4-byte aligned inputs
 * (bfloat16 value-typed fields: 2-byte); krec 16-byte aligned; for P > 1 every local slot of a
 * stream is < stream_offset.
 * Floating outputs agree with the exact (real-arithmetic) values within
 * max(1e-5 |value|, 1e-6); integer outputs are exact. A bfloat16 output is one of the two bfloat16
 * values next to the exact value (its float32 evaluation may fall on the other side of a rounding
 * midpoint), and so is the cpe in krec.
 */
sdm_status sdm_phase1(const sdm_p1_shape* shape, const sdm_p1_io* io, hipStream_t st);

/*
 * The pair sums A and QK of a Phase-1 call made with defer_pairs = 1 (page
 * "sparse_delta_memory/cuda/phase1_cuda.py": the pair kernels of its kernel plan, the same sums as
 * an sdm_phase1 call that computes them). `shape` and `io` are those of that call (the same
 * workspace, a and qk; at least one of a and qk set); st must be ordered after the call's stream
 * (an event, or the same stream), and the workspace must not be given to another sdm_phase1 call
 * until this call's kernel has run. Outputs and refusals as in sdm_phase1 (any non-zero status:
 * nothing was launched).
 */
sdm_status sdm_phase1_pairs(const sdm_p1_shape* shape, const sdm_p1_io* io, hipStream_t st);

/* One DW step: the chunks ti*P .. ti*P + P - 1 of the Phase-1 records. */
typedef struct sdm_dw_io {
    void* bank;             /* [rows, hd] SDM_F32 or SDM_BF16 bank, updated IN PLACE; 16-byte aligned when
                               hd is a vector width (below), else element-aligned */
    int32_t bank_dtype;     /* sdm_dtype */
    int64_t rows;           /* bank rows; every record slot is < rows */
    int32_t hd;             /* row width, 1..1024. Multiples of 8 up to 512 and of 16 up to 1024 take 16-byte
                               vector accesses; any other width takes element accesses (the mover pages'
                               scalar tail variant: same values and roundings, element-aligned rows) */
    const void* dv;         /* token rows: row (ti * dv_step_rows + p * C + t) of [*, hd]; aligned as bank */
    int32_t dv_dtype;       /* sdm_dtype (bf16 rows are widened exactly) */
    int64_t dv_step_rows;   /* rows between steps in dv (P*C when every step is stored, 0 for one step) */
    int64_t dv_rows;        /* rows in dv; ti * dv_step_rows + P * C <= dv_rows */
    const int32_t* krec;    /* [N, C*W, 4] records from sdm_phase1 */
    int32_t P, C, W, N;     /* the Phase-1 shape of krec */
    void* workspace;        /* optional (NULL: every group is walked by one team of lanes): device
                               memory of sdm_dw_workspace() bytes, 16-byte aligned, ZERO-FILLED before
                               its first use; every call leaves it zero-filled where it must be. With it,
                               groups longer than 32 members are split into 32-member segments summed
                               in parallel and combined in segment order. Calls sharing one workspace
                               must not run concurrently. */
    size_t workspace_bytes;
    hipEvent_t* events;     /* optional (NULL: none): 2 caller-created events bound to the start and end
                               of this call's kernel (hipExtLaunchKernel) */
    void* snap;             /* optional (NULL: none) compact snapshot, [*, hd] (snap_dtype), aligned
                               as bank: for every valid group of chunk ti*P + p whose FIRST is at K-row
                               position j, row (ti * snap_step_rows + p * C * W + j) receives the group's
                               pre-write bank row (page "sparse_delta_memory/cuda/mover_da2_cuda.py", the
                               da2_dw kernel's compact snapshot; page "sparse_delta_memory/cuda/mover_fx_cuda.py",
                               module docstring: the saving forward's raw copies of the base rows). Other rows
                               are not written. */
    int64_t snap_step_rows; /* rows between steps in snap (P*C*W when every step is kept, 0 for one step) */
    int64_t snap_rows;      /* rows in snap: ti * snap_step_rows + P * C * W <= snap_rows */
    int32_t snap_dtype;     /* element type of snap (sdm_dtype): the bank's own type gives the raw copy;
                               SDM_BF16 with an SDM_F32 bank gives each row rounded to bf16, nearest even (page
                               "sparse_delta_memory/cuda/mover_fx_cuda.py": the bf16 compact rows of a float32
                               bank); SDM_F32 rows of a bf16 bank are refused */
    const int32_t* snap_ord; /* optional (NULL: rows at FIRST positions, as above): gord_k from sdm_phase1; the
                               group whose FIRST is at K-row position j then goes to row (ti * snap_step_rows +
                               p * C * W + snap_ord[(ti*P + p) * C * W + j]), the dense layout: each chunk's
                               groups in rows 0 .. groups - 1 of its C * W rows */
} sdm_dw_io;

/* Workspace bytes sdm_dw_step can use for this shape: per block of 32 K-row positions of the step
   (B = ceil(P * C * W / 32) blocks) an arrival counter and a metadata pair (12 B) and two float32
   partial rows (8 hd B), each region rounded up to 256 bytes. */
size_t sdm_dw_workspace(const sdm_dw_io* io);

/*
 * DW decay-and-write (page "sparse_delta_memory/cuda/mover_da2_cuda.py", module docstring; bit
 * contract of "sparse_delta_memory/cuda/mover_fx_cuda.py", module docstring): for every valid
 * group of the K-only rows of chunks ti*P + p (p < P), in sorted order,
 *   acc = fma(sc_m, dv[token_m], acc) over the members from +0,
 *   bank[slot] = fma(bank[slot], cpe_last, acc)  (bf16 bank: rounded to nearest even).
 * With a workspace, a group longer than 32 members is summed as 32-member segment partials (each
 * an fma chain from +0) added in segment order, then the same final fma.
 * Rows of slots without a valid group are not touched. Within one call every slot has at most
 * one writer (stream slot ranges must not overlap). bank must not alias dv or krec.
 * Requires (ti + 1) * P <= N and ti * dv_step_rows + P * C <= dv_rows. A record whose slot is
 * >= rows is skipped (its group writes nothing).
 */
sdm_status sdm_dw_step(const sdm_dw_io* io, int64_t ti, hipStream_t st);

/*
 * sdm_dw_step for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same step, the same kernels and the same
 * bits as sdm_dw_step with a workspace, but the split-group workspace is a fixed 16 MiB array
 * inside the library (one copy per device, held until the process ends). io->workspace must be
 * NULL. Each call first clears the counters it uses (a small fill kernel on st), then enqueues the
 * step; it calls no allocating routine. Limits: P*C*W <= 4194304 K-row positions per step, and
 * 8 * hd * ceil(P*C*W / 32) bytes of partial rows <= 14.5 MiB (every workload shape up to
 * P*C*W = 131072 at hd = 128, or 8192 at hd = 960, fits); larger steps are refused with
 * SDM_EWORKSPACE before anything is enqueued. All calls on one device share the array: calls
 * that may overlap on one device (different streams without ordering, several host threads)
 * race and must be serialized by the caller.
 */
sdm_status sdm_dw_step_noalloc(const sdm_dw_io* io, int64_t ti, hipStream_t st);

/* One read-side step: the chunks ti*P .. ti*P + P - 1, before their DW step. */
typedef struct sdm_read_io {
    const void* bank;       /* [rows, hd] SDM_F32 or SDM_BF16: the memory BEFORE this step's DW (read only) */
    int32_t bank_dtype;     /* sdm_dtype */
    int64_t rows;           /* bank rows, >= 1 (an id outside 0..rows-1 contributes nothing) */
    int32_t hd;             /* row width, 1..4096 (a multiple of 8 takes 16-byte vector rows; any other
                               width element accesses, with element-aligned arrays) */
    const void* k_idx;      /* [N, C, W] absolute slot ids of the writes (Phase-1 input), int32 or int64 */
    const void* q_idx;      /* [N, C, R] absolute slot ids of the reads, same type */
    const void* k_eff;      /* [N, C, W] from sdm_phase1, float32 or bfloat16 (val_bytes) */
    const void* q_w;        /* [N, C, R] from sdm_phase1, same type */
    const float* a;         /* [N, C, C] from sdm_phase1 */
    const float* qk;        /* [N, C, C] from sdm_phase1 */
    const float* v;         /* value rows: row (ti * step_rows + p * C + t) of [*, hd], float32 */
    const float* beta;      /* [N, C] per-token write strengths */
    float* dv;              /* OUT token rows, same row indexing as v: feed sdm_dw_step (dv_step_rows =
                               step_rows, dv_dtype SDM_F32) */
    float* pred;            /* OUT predictions, same row indexing (also the call's scratch) */
    float* read;            /* OUT reads, same row indexing (also the call's scratch) */
    int64_t step_rows;      /* rows between steps in v / dv / pred / read (P*C, or 0 for one-step buffers) */
    int64_t out_rows;       /* rows in each of v, dv, pred and read: ti * step_rows + P * C <= out_rows */
    int32_t P, C, W, R, N;  /* the Phase-1 shape */
    int32_t first_partial;  /* as in sdm_p1_shape: tokens >= valid_last of chunks >= first_partial are masked */
    int32_t valid_last;
    int32_t idx_bytes;      /* width of k_idx / q_idx: 0 or 4 = int32, 8 = int64 */
    int32_t val_bytes;      /* type of k_eff / q_w as sdm_phase1 wrote them: 0 or 4 = float32, 2 = bfloat16 */
    hipEvent_t* events;     /* optional (NULL: none): 4 caller-created events bound to the start and end of
                               the gather kernel ([0], [1]) and of the substitution kernel ([2], [3]) */
} sdm_read_io;

/*
 * Forward read side of one step (definitions: page "sparse_delta_memory/cuda/phase1_cuda.py",
 * module docstring, for k_eff, q_w, A, QK; the delta rule dv = beta (v - prediction) as the write
 * scale -beta k exp(log_k) of the backward records on the same page, p1_scan_kernel, and on page
 * "sparse_delta_memory/cuda/pa_dc_cuda.py", module docstring, implies). Per chunk, from the bank
 * rows M0 before the step:
 *   p0[t] = sum_e k_eff[t,e] M0[k_idx[t,e]],   q0[t] = sum_r q_w[t,r] M0[q_idx[t,r]],
 *   dv[t] = beta[t] (v[t] - p0[t] - sum_{j<t} A[t,j] dv[j])    (forward substitution),
 *   pred[t] = p0[t] + sum_{j<t} A[t,j] dv[j],    read[t] = q0[t] + sum_{j<=t} QK[t,j] dv[j].
 * pred and read are what a token-by-token decay / predict / write / read evaluation of the chunk
 * sees; masked tokens get 0 in every output and none of their inputs is read. Two kernels on st.
 * Requires (ti + 1) * P <= N, C <= 256, 1 <= hd <= 4096; bank, v, dv, pred and read 16-byte aligned
 * when hd is a multiple of 8, element-aligned otherwise.
 */
sdm_status sdm_read_step(const sdm_read_io* io, int64_t ti, hipStream_t st);

/* GDS of one step: the backward of the read gather for the chunks ti*P .. ti*P + P - 1. */
typedef struct sdm_gds_io {
    const void* bank;       /* [rows, hd] SDM_F32 or SDM_BF16: the memory BEFORE this step's DW (read only) */
    int32_t bank_dtype;     /* sdm_dtype */
    int64_t rows;           /* bank rows, >= 1 (an id outside 0..rows-1 contributes nothing) */
    int32_t hd;             /* row width, a multiple of 4, 4..4096 */
    const void* q_idx;      /* [N, C, R] absolute slot ids of the reads (Phase-1 input), int32 or int64 */
    const void* q_w;        /* [N, C, R] from sdm_phase1, float32 or bf16 (val_bytes) */
    const int32_t* spay_q;  /* [N, C*R] Q-only row elements from sdm_phase1 */
    const float* gr;        /* gradient rows of the reads: row (ti * step_rows + p * C + t) of [*, hd], float32 */
    int64_t step_rows;      /* rows between steps in gr (P*C, or 0 for a one-step buffer) */
    int64_t gr_rows;        /* rows in gr: ti * step_rows + P * C <= gr_rows */
    float* d_q_w;           /* OUT (NULL: skipped) [N, C, R]: the chunks of step ti, 0 for masked tokens */
    void* grad;             /* IN/OUT (NULL: skipped) [rows, hd] SDM_F32 or SDM_BF16 gradient of the bank: every
                               slot a valid read of the step names gains its sum, one read-modify-write per
                               element (float32 add, then bf16 rounding to nearest even for a bf16 grad) */
    int32_t grad_dtype;     /* sdm_dtype */
    int32_t P, C, R, N;     /* the Phase-1 shape */
    int32_t first_partial;  /* as in sdm_p1_shape: tokens >= valid_last of chunks >= first_partial are masked */
    int32_t valid_last;
    int32_t idx_bytes;      /* width of q_idx: 0 or 4 = int32, 8 = int64 */
    int32_t val_bytes;      /* type of q_w: 0 or 4 = float32, 2 = bf16 */
    void* workspace;        /* optional (NULL: none), 16-byte aligned, sdm_gds_workspace(io) bytes, zero-filled
                               before its first use and left so by every call: read groups of more than 32
                               members are then summed in 32-member segments by separate waves, their partial
                               rows added in segment order by the last to finish (the same sums whichever
                               finishes last). Calls that share a workspace must not overlap. */
    size_t workspace_bytes;
} sdm_gds_io;

/*
 * GDS (page "sparse_delta_memory/cuda/mover_da2_cuda.py": the GDS part of the module docstring and
 * the comment of its scatter role): with the read gather q0[t] = sum_r q_w[t,r] M0[q_idx[t,r]] and
 * the gradient rows gr[t] of the reads,
 *   d_q_w[t, r] = <gr[t], M0[q_idx[t, r]]>                           (token order, no atomics),
 *   grad[s]    += sum over valid (t, r) with q_idx[t, r] = s of q_w[t, r] gr[t]
 * (sorted order: each valid Q group's members summed in order from +0, then one read-modify-write
 * of the slot's row by the group's only writer; results are reproducible run to run). Masked tokens
 * read nothing and contribute nothing. Within one step a slot appears in one group per chunk and
 * the P chunks' streams own disjoint slots, so the writes never overlap. Two kernels on st.
 * Requires (ti + 1) * P <= N, hd a multiple of 4, 16-byte aligned bank, gr and grad (8-byte for
 * bf16 rows), 4-byte aligned ids (8 for int64), q_w, spay_q and d_q_w.
 */
sdm_status sdm_gds_step(const sdm_gds_io* io, int64_t ti, hipStream_t st);

/* Bytes of the optional GDS workspace for this io's shape (P, C, R, hd): per block of 32 Q-row
 * positions of a step an arrival counter and a segment count (4 B each), and two float32 partial
 * rows. 0 for an invalid shape. */
size_t sdm_gds_workspace(const sdm_gds_io* io);

/* GWR of one step: the backward of DW's write terms for the tokens of chunks ti*P .. ti*P + P - 1. */
typedef struct sdm_gwr_io {
    const void* grad;       /* [rows, hd] SDM_F32 or SDM_BF16 gradient of the bank rows DW wrote (read only) */
    int32_t grad_dtype;     /* sdm_dtype */
    int64_t rows;           /* grad rows, >= 1 (an id outside 0..rows-1 contributes nothing) */
    int32_t hd;             /* row width, a multiple of 4, 4..1024 */
    const void* k_idx;      /* [N, C, W] absolute slot ids of the writes, int32 or int64 */
    const float* w;         /* [N, C, W] write weights (the DW scale k exp(rex) of each entry) */
    const float* dv;        /* token rows of the step: row (ti * step_rows + p * C + t) of [*, hd], float32 */
    int64_t step_rows;      /* rows between steps in dv and d_dv (P*C, or 0 for one-step buffers) */
    int64_t dv_rows;        /* rows in dv and d_dv: ti * step_rows + P * C <= dv_rows */
    float* d_dv;            /* OUT (NULL: skipped): rows in dv's layout, 0 for masked tokens */
    float* d_k_pd;          /* OUT (NULL: skipped) [N, C, W]: the chunks of step ti, 0 for masked tokens */
    int32_t P, C, W, N;     /* the Phase-1 shape */
    int32_t first_partial;  /* as in sdm_p1_shape */
    int32_t valid_last;
    int32_t idx_bytes;      /* width of k_idx: 0 or 4 = int32, 8 = int64 */
} sdm_gwr_io;

/*
 * GWR (page "sparse_delta_memory/cuda/pa_dc_cuda.py", module docstring: the GWR gather of the
 * deterministic backward step):
 *   d_dv[t]      = sum_n w[t, n] grad[k_idx[t, n]]     (the token's entries in order, from +0),
 *   d_k_pd[t, n] = <dv[t], grad[k_idx[t, n]]>.
 * Masked tokens get zeros and none of their inputs is read. One kernel on st; no atomics, so the
 * results are reproducible. Requires (ti + 1) * P <= N, hd a multiple of 4 up to 1024, 16-byte
 * aligned dv and d_dv, grad rows 16-byte aligned (8 for bf16), 4-byte aligned w, d_k_pd and ids
 * (8 for int64).
 */
sdm_status sdm_gwr_step(const sdm_gwr_io* io, int64_t ti, hipStream_t st);

/* PA of one step: the backward of DW for the write groups of chunks ti*P .. ti*P + P - 1. */
typedef struct sdm_pa_io {
    void* grad;             /* IN/OUT [rows, hd] SDM_F32 or SDM_BF16 bank gradient: each written slot's row
                               becomes gdw * cpe + sum_m sc_m d_dva[tok_m] (gdw: its value before the call) */
    int32_t grad_dtype;     /* sdm_dtype */
    void* bank;             /* OUT (NULL: skipped) [rows, hd]: each written slot's row restored from snap */
    int32_t bank_dtype;     /* sdm_dtype of bank and snap */
    int64_t rows;           /* rows of grad and bank, >= 1 (a slot outside 0..rows-1 is skipped) */
    int32_t hd;             /* row width, a multiple of 4, 4..1024 */
    const void* snap;       /* the step's compact snapshot from sdm_dw_step (FIRST-position layout, raw rows) */
    int64_t snap_step_rows; /* as given to sdm_dw_step */
    int64_t snap_rows;      /* rows in snap: ti * snap_step_rows + P * C * W <= snap_rows */
    const int32_t* krec;    /* [N, C*W, 4] records from sdm_phase1 */
    const void* k_eff;      /* [N, C, W] from sdm_phase1, float32 or bf16 (val_bytes) */
    const float* beta;      /* [N, C] per-token write strengths */
    const float* d_dva;     /* gradient token rows: row (ti * step_rows + p * C + t) of [*, hd], float32 */
    int64_t step_rows;      /* rows between steps in d_dva (P*C, or 0 for a one-step buffer) */
    int64_t dva_rows;       /* rows in d_dva: ti * step_rows + P * C <= dva_rows */
    float* g_decay;         /* OUT (NULL: skipped) [N, C, W]: grad_g_decay of the step's entries, 0 for padding */
    float* d_k_eff;         /* OUT (NULL: skipped) [N, C, W]: d_k_eff of the step's entries, 0 for padding */
    int32_t P, C, W, N;     /* the Phase-1 shape */
    int32_t val_bytes;      /* type of k_eff: 0 or 4 = float32, 2 = bf16 */
    void* workspace;        /* optional (NULL: every group is walked by one wave): device memory of
                               sdm_pa_workspace() bytes, 16-byte aligned, ZERO-FILLED before its first
                               use; every call leaves it zero-filled where it must be. With it, a group
                               longer than 32 members is split into 32-member segments walked by waves
                               of their own; the segments' partial sums are added in segment order by
                               the last segment to finish. Calls sharing one workspace must not run
                               concurrently. */
    size_t workspace_bytes;
} sdm_pa_io;

/* Workspace bytes sdm_pa_step can use for this shape: per block of 32 K-row positions of the step
   (B = ceil(P * C * W / 32) blocks) an arrival counter and a segment count (8 B) and two float32
   partial rows (8 hd B), each region rounded up to 256 bytes. */
size_t sdm_pa_workspace(const sdm_pa_io* io);

/*
 * PA (page "sparse_delta_memory/cuda/pa_dc_cuda.py", module docstring: Phase A of the deterministic
 * backward step): per valid write group (slot s, members m in sorted order), with gdw = grad[s]
 * before the call, snap the group's pre-write row and cpe the group's record cpe,
 *   grad[s]         = fma(gdw, cpe, sum_m sc_m d_dva[tok_m])   (sum from +0, sc_m = -beta k_eff_m),
 *   bank[s]         = snap,
 *   grad_g_decay[e] = cpe <gdw, snap>,   d_k_eff[e] = -beta[tok_e] <d_dva[tok_e], snap>.
 * With a workspace, a group longer than 32 members sums sc_m d_dva[tok_m] per 32-member segment
 * (each from +0) and adds the partials in segment order before the final fma.
 * One writer per row and per entry, fixed sum orders: reproducible. Padding entries get
 * zeros; masked tokens' rows are never read. Requires (ti + 1) * P <= N, hd a multiple of 4 up to
 * 1024, 16-byte aligned grad, bank, snap and d_dva rows (8 for bf16 rows), 16-byte aligned krec.
 */
sdm_status sdm_pa_step(const sdm_pa_io* io, int64_t ti, hipStream_t st);

/* Static text for a status code. */
const char* sdm_status_string(sdm_status s);

/* Message of the last failed call on this thread ("" if none). */
const char* sdm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SDM_H */
