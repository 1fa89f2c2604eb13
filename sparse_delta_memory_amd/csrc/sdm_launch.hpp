// Host-side launch interface between the C ABI (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "sdm.h"

namespace sdm {

// Longest chunk row (C * (W + R)) one Phase-1 workgroup sorts and scans on chip; longer rows (up
// to 2^17 entries) take the tiled path.
constexpr int kP1MaxRow = 16384;
constexpr int kP1MaxTiledRow = 1 << 17;
constexpr int kP1Threads = 1024;

// Valid K entries that make a slot group "hot": the pair kernel sums such groups densely.
constexpr int kHotMin = 16;

// Kernels launched with dynamic LDS, each file listing its own (fills fns, returns the count, at
// most cap). The ABI raises their dynamic-LDS limit to the device's maximum once per device, before
// the first launch there, so no launch sequence makes another runtime call between its kernels.
int p1_lds_kernels(const void** fns, int cap);
int read_lds_kernels(const void** fns, int cap);

// The kernel a Phase-1 launch sequence was enqueuing when it failed (for the error message).
extern thread_local const char* g_p1_stage;

struct P1Launch {
    const sdm_p1_shape* s;
    const sdm_p1_io* io;
    void* rec;        // [N, n] 16-byte records in sorted order: payload | head, log-cumsum (s, c), value
    void* inv_k;      // [N, C*W] uint16 per K entry (entry order): sorted position (bits 0-13), bit 15
                      // where the entry starts its token's run with earlier valid K entries of an
                      // ordinary (not hot) group
    void* inv_q;      // [N, C*R] the same for the Q entries
    void* hot;        // [N, hot_cap + 1] uint2: count, then {head position, size} of each hot group
    void* sort;       // tiled path: [N, 4, n] uint32 key and entry-index buffers (two of each)
    void* rev;        // tiled path: [N, n, 3] uint32 reverse-scan results per sorted position
    int lds_max;      // LDS bytes per block of the device
};

// The pair kernel's plan: hot groups per chunk, groups per batch, blocks per compute unit, and
// whether hot groups are summed densely (the Phase-1 kernels then list them).
struct PairPlan {
    int hot_cap, gb, blocks_cu;
    bool hot_on;
};
PairPlan pair_plan(const sdm_p1_shape* s, bool pairs, int lds_max);
// The pair kernel on st (inv32: 32-bit entry-order words of the tiled path).
hipError_t pair_launch(const P1Launch& L, const PairPlan& pp, bool inv32, hipStream_t st);
// The dense group ordinals (gord_k) on st, when asked for.
hipError_t p1_ordinal_launch(const sdm_p1_shape* s, const sdm_p1_io* io, hipStream_t st);
// The tiled path: its kernel, then the ordinals and the pair kernel.
hipError_t p1_tiled_launch(const P1Launch& L, hipStream_t st);
size_t p1_tiled_lds_bytes(const sdm_p1_shape* s);
int p1_tiled_lds_kernels(const void** fns, int cap);

// Workspace layout of sdm_phase1: byte offsets of the regions and the total. The tiled path
// (rows longer than kP1MaxRow, or shape->tiled) adds its sort buffers and reverse-scan results and
// keeps 32-bit entry-order pair words.
struct P1Workspace {
    size_t rec_off, inv_k_off, inv_q_off, hot_off, sort_off, rev_off, total;
    int hot_cap;      // hot groups a chunk can hold: C * W / kHotMin
    bool tiled;
};
P1Workspace p1_workspace_layout(const sdm_p1_shape* s);

// Whether a shape goes through the tiled (long-row) path.
bool p1_tiled(const sdm_p1_shape* s);

// Dynamic LDS bytes of the Phase-1 sort/scan kernel for this shape and output set.
size_t p1_lds_bytes(const sdm_p1_shape* s, const sdm_p1_io* io);

// LDS bytes the pair kernel needs without hot-group tables (the triangle and the hot list).
size_t p1_pair_lds_min(const sdm_p1_shape* s);

// Enqueue the Phase-1 kernels; returns hipSuccess or the first launch error. With io->defer_pairs the
// pair kernel is left out (its inputs are still written) for p1_pairs_launch.
hipError_t p1_launch(const P1Launch& L, hipStream_t st);
// The pair kernel alone, from the workspace of an earlier p1_launch of the same shape and io.
hipError_t p1_pairs_launch(const P1Launch& L, hipStream_t st);

struct DwLaunch {
    const sdm_dw_io* io;
    int64_t ti;
};

hipError_t dw_launch(const DwLaunch& L, hipStream_t st);

// Allocation-free DW: the split workspace in the library's fixed device array. dw_static_fits says
// whether a step of this shape fits it (need / cap: partial-row bytes); dw_static_setup finds the
// array's address on the current device (once per device); dw_launch_static clears the call's
// counters with a fill kernel and enqueues the step.
bool dw_static_fits(const sdm_dw_io* io, size_t* need, size_t* cap);
hipError_t dw_static_setup();
hipError_t dw_launch_static(const DwLaunch& L, hipStream_t st);

// Workspace of sdm_dw_step: per block of 32 K-row positions an arrival counter (zero between
// calls) and group metadata, and two partial rows.
struct DwWorkspace {
    size_t cnt_off, cnt_bytes, meta_off, part_off, total;
};
DwWorkspace dw_workspace_layout(const sdm_dw_io* io);

struct ReadLaunch {
    const sdm_read_io* io;
    int64_t ti;
};

// Enqueue the read side of one step (gather kernel, then substitution kernel).
hipError_t read_launch(const ReadLaunch& L, hipStream_t st);

// GDS of step ti (validated by sdm_gds_step).
hipError_t gds_launch(const sdm_gds_io* io, int64_t ti, hipStream_t st);

// Workspace of sdm_gds_step: per block of 32 Q-row positions an arrival counter (zero between
// calls) and a segment count, and two partial rows.
struct GdsWorkspace {
    size_t cnt_off, meta_off, part_off, total;
};
GdsWorkspace gds_workspace_layout(const sdm_gds_io* io);

// GWR of step ti (validated by sdm_gwr_step).
hipError_t gwr_launch(const sdm_gwr_io* io, int64_t ti, hipStream_t st);

// PA of step ti (validated by sdm_pa_step).
hipError_t pa_launch(const sdm_pa_io* io, int64_t ti, hipStream_t st);

// Workspace of sdm_pa_step: per block of 32 K-row positions an arrival counter (zero between
// calls) and a segment count, and two partial rows.
struct PaWorkspace {
    size_t cnt_off, meta_off, part_off, total;
};
PaWorkspace pa_workspace_layout(const sdm_pa_io* io);

}  // namespace sdm
