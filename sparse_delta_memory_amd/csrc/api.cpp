// C ABI of the SDM forward hot path: argument checks on the host, then the kernel launches.
// Preconditions follow the pages' host launchers ("sparse_delta_memory/cuda/mover_da2_cuda.py",
// da2_dw: C <= 256, 16-byte rows and alignment; "sparse_delta_memory/cuda/phase1_cuda.py": 8-bit
// token and lane fields, 17-bit positions) restated for this implementation.
#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <mutex>
#include <string>

#include "sdm.h"
#include "sdm_launch.hpp"

namespace sdm {
int dw_cols_per_lane(int hd);
bool dw_tail(int hd);
}

namespace {

thread_local std::string g_last_error;

sdm_status fail(sdm_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Once per device, before the first launch there: the device's LDS bytes per workgroup, and every
// dynamic-LDS kernel's limit raised to it. Entry points call this after their argument checks and
// before their first enqueue.
constexpr int kMaxDevices = 64;
struct DeviceSetup {
    std::once_flag once;
    hipError_t err = hipSuccess;
    int lds_max = 0;
};
DeviceSetup g_setup[kMaxDevices];

hipError_t device_setup(int* lds_max) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    DeviceSetup& d = g_setup[dev];
    std::call_once(d.once, [&d, dev]() {
        int lds = 0;
        d.err = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
        if (d.err != hipSuccess) return;
        const void* fns[128];
        int n = sdm::p1_lds_kernels(fns, 128);
        n += sdm::read_lds_kernels(fns + n, 128 - n);
        for (int i = 0; i < n && d.err == hipSuccess; ++i) {
            // The dynamic limit is what the device holds beside the kernel's static LDS.
            hipFuncAttributes fa;
            d.err = hipFuncGetAttributes(&fa, fns[i]);
            if (d.err != hipSuccess) break;
            const int dyn = lds - static_cast<int>(fa.sharedSizeBytes);
            if (dyn > 0) d.err = hipFuncSetAttribute(fns[i], hipFuncAttributeMaxDynamicSharedMemorySize, dyn);
        }
        if (d.err != hipSuccess) (void)hipGetLastError();   // reported through the status, not left pending
        d.lds_max = lds;
    });
    if (lds_max != nullptr) *lds_max = d.lds_max;
    return d.err;
}

sdm_status check_p1_shape(const sdm_p1_shape* s) {
    if (s == nullptr) return fail(SDM_EINVAL, "sdm_phase1: shape is NULL");
    if (s->N < 0) return fail(SDM_ESHAPE, "sdm_phase1: N = %d < 0", s->N);
    if (s->C < 1 || s->C > 256) return fail(SDM_ESHAPE, "sdm_phase1: C = %d outside 1..256", s->C);
    if (s->W < 1 || s->W > 256) return fail(SDM_ESHAPE, "sdm_phase1: W = %d outside 1..256", s->W);
    if (s->R < 1 || s->R > 256) return fail(SDM_ESHAPE, "sdm_phase1: R = %d outside 1..256", s->R);
    if (s->P < 1) return fail(SDM_ESHAPE, "sdm_phase1: P = %d < 1", s->P);
    if (s->key_bits < 1 || s->key_bits > 30) return fail(SDM_EINVAL, "sdm_phase1: key_bits = %d outside 1..30", s->key_bits);
    if (s->stream_offset < 0) return fail(SDM_EINVAL, "sdm_phase1: stream_offset < 0");
    if (s->first_partial < 0 || s->first_partial > s->N)
        return fail(SDM_EINVAL, "sdm_phase1: first_partial = %d outside 0..N", s->first_partial);
    if (s->valid_last < 0 || s->valid_last > s->C)
        return fail(SDM_EINVAL, "sdm_phase1: valid_last = %d outside 0..C", s->valid_last);
    if (s->tile_len < 1) return fail(SDM_EINVAL, "sdm_phase1: tile_len = %d < 1", s->tile_len);
    if (s->idx_bytes != 0 && s->idx_bytes != 4 && s->idx_bytes != 8)
        return fail(SDM_EINVAL, "sdm_phase1: idx_bytes = %d (0 or 4: int32 ids; 8: int64 ids)", s->idx_bytes);
    if (s->val_bytes != 0 && s->val_bytes != 4 && s->val_bytes != 2)
        return fail(SDM_EINVAL, "sdm_phase1: val_bytes = %d (0 or 4: float32 values; 2: bfloat16)", s->val_bytes);
    if (s->g_lane_stride != 0 && s->g_lane_stride != 1)
        return fail(SDM_EINVAL, "sdm_phase1: g_lane_stride = %d (0: gates [N, C]; 1: gates [N, C, W])", s->g_lane_stride);
    const int64_t n = static_cast<int64_t>(s->C) * (s->W + s->R);
    if (n > sdm::kP1MaxTiledRow) return fail(SDM_ESHAPE, "sdm_phase1: C*(W+R) = %lld > 2^17", static_cast<long long>(n));
    if (s->tiled != 0 && s->tiled != 1) return fail(SDM_EINVAL, "sdm_phase1: tiled = %d (0 or 1)", s->tiled);
    if (s->lds_budget != 0 && (s->lds_budget < 16384 || s->lds_budget > 163840))
        return fail(SDM_EINVAL, "sdm_phase1: lds_budget = %d (0, or 16384..163840)", s->lds_budget);
    if (s->pair_walk != 0 && s->pair_walk != 1) return fail(SDM_EINVAL, "sdm_phase1: pair_walk = %d (0 or 1)", s->pair_walk);
    return SDM_OK;
}

sdm_status check_dw_io(const sdm_dw_io* io, int64_t ti, const char* fn) {
    if (io->C < 1 || io->C > 256 || io->W < 1 || io->W > 256)
        return fail(SDM_ESHAPE, "%s: C = %d, W = %d outside 1..256", fn, io->C, io->W);
    if (io->P < 1 || io->N < 0) return fail(SDM_ESHAPE, "%s: P = %d, N = %d", fn, io->P, io->N);
    if (static_cast<int64_t>(io->P) * io->C * io->W > (int64_t(1) << 30))
        return fail(SDM_ESHAPE, "%s: P*C*W = %lld > 2^30 positions per step", fn,
                    static_cast<long long>(static_cast<int64_t>(io->P) * io->C * io->W));
    if (ti < 0 || (ti + 1) * static_cast<int64_t>(io->P) > io->N)
        return fail(SDM_ESHAPE, "%s: step %lld needs (ti+1)*P <= N = %d", fn, static_cast<long long>(ti), io->N);
    if (io->bank_dtype != SDM_F32 && io->bank_dtype != SDM_BF16)
        return fail(SDM_EINVAL, "%s: bank_dtype %d", fn, io->bank_dtype);
    if (io->dv_dtype != SDM_F32 && io->dv_dtype != SDM_BF16)
        return fail(SDM_EINVAL, "%s: dv_dtype %d", fn, io->dv_dtype);
    if (io->hd < 1 || io->hd > 4096) return fail(SDM_ESHAPE, "%s: hd = %d outside 1..4096", fn, io->hd);
    if (sdm::dw_cols_per_lane(io->hd) == 0)
        return fail(SDM_EUNSUPPORTED, "%s: hd = %d (this build: up to 1024)", fn, io->hd);
    if (io->rows < 1 || io->dv_step_rows < 0 || io->dv_rows < 0)
        return fail(SDM_EINVAL, "%s: rows / dv_step_rows / dv_rows", fn);
    if (ti * io->dv_step_rows + static_cast<int64_t>(io->P) * io->C > io->dv_rows)
        return fail(SDM_EINVAL, "%s: dv holds %lld rows, step %lld needs %lld", fn, static_cast<long long>(io->dv_rows),
                    static_cast<long long>(ti), static_cast<long long>(ti * io->dv_step_rows + static_cast<int64_t>(io->P) * io->C));
    if (io->bank == nullptr || io->dv == nullptr || io->krec == nullptr)
        return fail(SDM_EINVAL, "%s: bank, dv and krec are required", fn);
    // Head dims that 16-byte vectors divide (multiples of 8 up to 512, of 16 up to 1024) use vector
    // accesses and need 16-byte aligned rows; any other takes element accesses (element alignment).
    const bool tail = sdm::dw_tail(io->hd);
    const int bank_es = io->bank_dtype == SDM_BF16 ? 2 : 4;
    const int dv_es = io->dv_dtype == SDM_BF16 ? 2 : 4;
    if (!aligned(io->krec, 16)) return fail(SDM_EALIGN, "%s: krec must be 16-byte aligned", fn);
    if (!aligned(io->bank, tail ? bank_es : 16) || !aligned(io->dv, tail ? dv_es : 16))
        return fail(SDM_EALIGN, "%s: bank and dv must be %s aligned", fn, tail ? "element" : "16-byte");
    if (io->workspace != nullptr) {
        if (!aligned(io->workspace, 16)) return fail(SDM_EALIGN, "%s: workspace is not 16-byte aligned", fn);
        const size_t need = sdm::dw_workspace_layout(io).total;
        if (io->workspace_bytes < need)
            return fail(SDM_EWORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, need, io->workspace_bytes);
    }
    if (io->snap != nullptr) {
        if (io->snap_dtype != io->bank_dtype && !(io->snap_dtype == SDM_BF16 && io->bank_dtype == SDM_F32))
            return fail(SDM_EINVAL, "%s: snap_dtype %d (the bank's, or bf16 rows of a float32 bank)", fn,
                        io->snap_dtype);
        if (!aligned(io->snap_ord, 4)) return fail(SDM_EALIGN, "%s: snap_ord is misaligned", fn);
        const int snap_es = io->snap_dtype == SDM_BF16 ? 2 : bank_es;
        if (!aligned(io->snap, tail ? snap_es : 16)) return fail(SDM_EALIGN, "%s: snap is misaligned", fn);
        const int64_t pcw = static_cast<int64_t>(io->P) * io->C * io->W;
        if (io->snap_step_rows < 0 || ti * io->snap_step_rows + pcw > io->snap_rows)
            return fail(SDM_EINVAL, "%s: snap holds %lld rows, step %lld needs %lld", fn,
                        static_cast<long long>(io->snap_rows), static_cast<long long>(ti),
                        static_cast<long long>(ti * io->snap_step_rows + pcw));
    }
    return SDM_OK;
}

}  // namespace

extern "C" {

const char* sdm_status_string(sdm_status s) {
    switch (s) {
        case SDM_OK: return "ok";
        case SDM_EINVAL: return "invalid argument";
        case SDM_ESHAPE: return "shape outside the supported ranges";
        case SDM_EALIGN: return "misaligned pointer";
        case SDM_EUNSUPPORTED: return "shape not implemented by this build";
        case SDM_EWORKSPACE: return "workspace missing or too small";
        case SDM_EHIP: return "HIP error";
    }
    return "unknown status";
}

const char* sdm_last_error(void) { return g_last_error.c_str(); }

size_t sdm_dw_workspace(const sdm_dw_io* io) {
    if (io == nullptr || io->P < 1 || io->C < 1 || io->W < 1 || io->hd < 1) return 0;
    return sdm::dw_workspace_layout(io).total;
}

size_t sdm_gds_workspace(const sdm_gds_io* io) {
    if (io == nullptr || io->P < 1 || io->C < 1 || io->R < 1 || io->hd < 1) return 0;
    return sdm::gds_workspace_layout(io).total;
}

size_t sdm_pa_workspace(const sdm_pa_io* io) {
    if (io == nullptr || io->P < 1 || io->C < 1 || io->W < 1 || io->hd < 1) return 0;
    return sdm::pa_workspace_layout(io).total;
}

size_t sdm_phase1_workspace(const sdm_p1_shape* s) {
    if (check_p1_shape(s) != SDM_OK) return 0;
    return sdm::p1_workspace_layout(s).total;
}

sdm_status sdm_phase1(const sdm_p1_shape* s, const sdm_p1_io* io, hipStream_t st) {
    g_last_error.clear();
    sdm_status rc = check_p1_shape(s);
    if (rc != SDM_OK) return rc;
    if (io == nullptr) return fail(SDM_EINVAL, "sdm_phase1: io is NULL");
    if (s->N == 0) return SDM_OK;
    const void* req[] = {io->k_idx, io->q_idx, io->k_val, io->q_val, io->g, io->spay_k, io->krec, io->tiles_k};
    const char* req_names[] = {"k_idx", "q_idx", "k_val", "q_val", "g", "spay_k", "krec", "tiles_k"};
    for (int i = 0; i < 8; ++i) {
        if (req[i] == nullptr) return fail(SDM_EINVAL, "sdm_phase1: %s is NULL", req_names[i]);
    }
    const void* a4[] = {io->k_idx, io->q_idx, io->g, io->log_k, io->rex, io->pos_k, io->log_q, io->pos_q,
                        io->spay_k, io->spay_q, io->tiles_k, io->a, io->qk, io->repeats, io->perm, io->status,
                        io->gord_k};
    for (const void* p : a4) {
        if (!aligned(p, 4)) return fail(SDM_EALIGN, "sdm_phase1: a 4-byte field is misaligned");
    }
    const void* av[] = {io->k_val, io->q_val, io->cpe, io->k_eff, io->q_w};   // value-typed fields
    for (const void* p : av) {
        if (!aligned(p, s->val_bytes == 2 ? 2 : 4)) return fail(SDM_EALIGN, "sdm_phase1: a value-typed field is misaligned");
    }
    if (!aligned(io->krec, 16)) return fail(SDM_EALIGN, "sdm_phase1: krec is not 16-byte aligned");
    if (s->idx_bytes == 8 && (!aligned(io->k_idx, 8) || !aligned(io->q_idx, 8)))
        return fail(SDM_EALIGN, "sdm_phase1: int64 ids must be 8-byte aligned");
    const sdm::P1Workspace ws = sdm::p1_workspace_layout(s);
    if (io->workspace == nullptr || io->workspace_bytes < ws.total)
        return fail(SDM_EWORKSPACE, "sdm_phase1: workspace needs %zu bytes, got %zu", ws.total,
                    io->workspace == nullptr ? size_t(0) : io->workspace_bytes);
    if (!aligned(io->workspace, 16)) return fail(SDM_EALIGN, "sdm_phase1: workspace is not 16-byte aligned");
    if (io->defer_pairs != 0 && io->defer_pairs != 1)
        return fail(SDM_EINVAL, "sdm_phase1: defer_pairs = %d (0 or 1)", io->defer_pairs);
    if (io->defer_pairs == 1 && io->a == nullptr && io->qk == nullptr)
        return fail(SDM_EINVAL, "sdm_phase1: defer_pairs = 1 without a or qk");
    const size_t main_lds = sdm::p1_lds_bytes(s, io);
    if (main_lds == SIZE_MAX)
        return fail(SDM_EUNSUPPORTED, "sdm_phase1: the sort/scan kernel's plan does not fit the LDS budget of %d B",
                    s->lds_budget);
    int lds_max = 0;
    const hipError_t se = device_setup(&lds_max);
    if (se != hipSuccess) return fail(SDM_EHIP, "sdm_phase1: device set-up: %s", hipGetErrorString(se));
    if (main_lds > static_cast<size_t>(lds_max))
        return fail(SDM_EUNSUPPORTED, "sdm_phase1: the sort/scan kernel needs %zu B of LDS per block, the device has %d",
                    main_lds, lds_max);
    const size_t tri = sdm::p1_pair_lds_min(s);
    if ((io->a != nullptr || io->qk != nullptr) && tri > static_cast<size_t>(lds_max))
        return fail(SDM_EUNSUPPORTED, "sdm_phase1: the C=%d pair kernel (%zu B) exceeds the %d B of LDS per block", s->C,
                    tri, lds_max);
    sdm::P1Launch L;
    L.s = s;
    L.io = io;
    L.rec = static_cast<char*>(io->workspace) + ws.rec_off;
    L.inv_k = static_cast<char*>(io->workspace) + ws.inv_k_off;
    L.inv_q = static_cast<char*>(io->workspace) + ws.inv_q_off;
    L.hot = static_cast<char*>(io->workspace) + ws.hot_off;
    L.sort = ws.tiled ? static_cast<char*>(io->workspace) + ws.sort_off : nullptr;
    L.rev = ws.tiled ? static_cast<char*>(io->workspace) + ws.rev_off : nullptr;
    L.lds_max = lds_max;
    sdm::g_p1_stage = "";
    const hipError_t e = sdm::p1_launch(L, st);
    if (e != hipSuccess) {
        (void)hipGetLastError();   // the launch's error is reported through the status, not left pending
        return fail(SDM_EHIP, "sdm_phase1: %s: %s", sdm::g_p1_stage, hipGetErrorString(e));
    }
    return SDM_OK;
}

sdm_status sdm_phase1_pairs(const sdm_p1_shape* s, const sdm_p1_io* io, hipStream_t st) {
    g_last_error.clear();
    sdm_status rc = check_p1_shape(s);
    if (rc != SDM_OK) return rc;
    if (io == nullptr) return fail(SDM_EINVAL, "sdm_phase1_pairs: io is NULL");
    if (io->a == nullptr && io->qk == nullptr) return fail(SDM_EINVAL, "sdm_phase1_pairs: neither a nor qk is set");
    if (!aligned(io->a, 4) || !aligned(io->qk, 4)) return fail(SDM_EALIGN, "sdm_phase1_pairs: a or qk is misaligned");
    if (s->N == 0) return SDM_OK;
    const sdm::P1Workspace ws = sdm::p1_workspace_layout(s);
    if (io->workspace == nullptr || io->workspace_bytes < ws.total)
        return fail(SDM_EWORKSPACE, "sdm_phase1_pairs: workspace needs %zu bytes, got %zu", ws.total,
                    io->workspace == nullptr ? size_t(0) : io->workspace_bytes);
    if (!aligned(io->workspace, 16)) return fail(SDM_EALIGN, "sdm_phase1_pairs: workspace is not 16-byte aligned");
    int lds_max = 0;
    const hipError_t se = device_setup(&lds_max);
    if (se != hipSuccess) return fail(SDM_EHIP, "sdm_phase1_pairs: device set-up: %s", hipGetErrorString(se));
    const size_t tri = sdm::p1_pair_lds_min(s);
    if (tri > static_cast<size_t>(lds_max))
        return fail(SDM_EUNSUPPORTED, "sdm_phase1_pairs: the C=%d pair kernel (%zu B) exceeds the %d B of LDS per block",
                    s->C, tri, lds_max);
    sdm::P1Launch L;
    L.s = s;
    L.io = io;
    L.rec = static_cast<char*>(io->workspace) + ws.rec_off;
    L.inv_k = static_cast<char*>(io->workspace) + ws.inv_k_off;
    L.inv_q = static_cast<char*>(io->workspace) + ws.inv_q_off;
    L.hot = static_cast<char*>(io->workspace) + ws.hot_off;
    L.sort = nullptr;
    L.rev = nullptr;
    L.lds_max = lds_max;
    const hipError_t e = sdm::p1_pairs_launch(L, st);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(SDM_EHIP, "sdm_phase1_pairs: pair kernel: %s", hipGetErrorString(e));
    }
    return SDM_OK;
}

sdm_status sdm_read_step(const sdm_read_io* io, int64_t ti, hipStream_t st) {
    g_last_error.clear();
    if (io == nullptr) return fail(SDM_EINVAL, "sdm_read_step: io is NULL");
    if (io->C < 1 || io->C > 256 || io->W < 1 || io->W > 256 || io->R < 1 || io->R > 256)
        return fail(SDM_ESHAPE, "sdm_read_step: C = %d, W = %d, R = %d outside 1..256", io->C, io->W, io->R);
    if (io->P < 1 || io->N < 0) return fail(SDM_ESHAPE, "sdm_read_step: P = %d, N = %d", io->P, io->N);
    if (ti < 0 || (ti + 1) * static_cast<int64_t>(io->P) > io->N)
        return fail(SDM_ESHAPE, "sdm_read_step: step %lld needs (ti+1)*P <= N = %d", static_cast<long long>(ti), io->N);
    if (io->first_partial < 0 || io->first_partial > io->N || io->valid_last < 0 || io->valid_last > io->C)
        return fail(SDM_EINVAL, "sdm_read_step: first_partial = %d, valid_last = %d", io->first_partial, io->valid_last);
    if (io->bank_dtype != SDM_F32 && io->bank_dtype != SDM_BF16)
        return fail(SDM_EINVAL, "sdm_read_step: bank_dtype %d", io->bank_dtype);
    if (io->idx_bytes != 0 && io->idx_bytes != 4 && io->idx_bytes != 8)
        return fail(SDM_EINVAL, "sdm_read_step: idx_bytes = %d (0 or 4: int32 ids; 8: int64 ids)", io->idx_bytes);
    if (io->val_bytes != 0 && io->val_bytes != 4 && io->val_bytes != 2)
        return fail(SDM_EINVAL, "sdm_read_step: val_bytes = %d (0 or 4: float32 k_eff / q_w; 2: bfloat16)", io->val_bytes);
    if (io->idx_bytes == 8 && (!aligned(io->k_idx, 8) || !aligned(io->q_idx, 8)))
        return fail(SDM_EALIGN, "sdm_read_step: int64 ids must be 8-byte aligned");
    if (io->hd < 1 || io->hd > 4096) return fail(SDM_ESHAPE, "sdm_read_step: hd = %d outside 1..4096", io->hd);
    if (io->rows < 1 || io->step_rows < 0 || io->out_rows < 0)
        return fail(SDM_EINVAL, "sdm_read_step: rows / step_rows / out_rows");
    if (ti * io->step_rows + static_cast<int64_t>(io->P) * io->C > io->out_rows)
        return fail(SDM_EINVAL, "sdm_read_step: %lld rows, step %lld needs %lld", static_cast<long long>(io->out_rows),
                    static_cast<long long>(ti), static_cast<long long>(ti * io->step_rows + static_cast<int64_t>(io->P) * io->C));
    const void* req[] = {io->bank, io->k_idx, io->q_idx, io->k_eff, io->q_w, io->a, io->qk, io->v, io->beta,
                         io->dv, io->pred, io->read};
    for (const void* p : req) {
        if (p == nullptr) return fail(SDM_EINVAL, "sdm_read_step: every array is required");
    }
    // hd a multiple of 8: 16-byte vector rows; any other hd: element accesses (element alignment).
    const bool tail = io->hd % 8 != 0;
    const void* a16[] = {io->bank, io->v, io->dv, io->pred, io->read};
    const uintptr_t es[] = {static_cast<uintptr_t>(io->bank_dtype == SDM_BF16 ? 2 : 4), 4, 4, 4, 4};
    for (int i = 0; i < 5; ++i) {
        if (!aligned(a16[i], tail ? es[i] : 16))
            return fail(SDM_EALIGN, "sdm_read_step: bank, v, dv, pred and read must be %s aligned",
                        tail ? "element" : "16-byte");
    }
    const void* a4[] = {io->k_idx, io->q_idx, io->a, io->qk, io->beta};
    for (const void* p : a4) {
        if (!aligned(p, 4)) return fail(SDM_EALIGN, "sdm_read_step: a 4-byte field is misaligned");
    }
    if (!aligned(io->k_eff, io->val_bytes == 2 ? 2 : 4) || !aligned(io->q_w, io->val_bytes == 2 ? 2 : 4))
        return fail(SDM_EALIGN, "sdm_read_step: k_eff / q_w misaligned for their type");
    const hipError_t se = device_setup(nullptr);
    if (se != hipSuccess) return fail(SDM_EHIP, "sdm_read_step: device set-up: %s", hipGetErrorString(se));
    sdm::ReadLaunch L;
    L.io = io;
    L.ti = ti;
    const hipError_t e = sdm::read_launch(L, st);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(SDM_EHIP, "sdm_read_step: %s", hipGetErrorString(e));
    }
    return SDM_OK;
}

sdm_status sdm_gds_step(const sdm_gds_io* io, int64_t ti, hipStream_t st) {
    g_last_error.clear();
    if (io == nullptr) return fail(SDM_EINVAL, "sdm_gds_step: io is NULL");
    if (io->C < 1 || io->C > 256 || io->R < 1 || io->R > 256)
        return fail(SDM_ESHAPE, "sdm_gds_step: C = %d, R = %d outside 1..256", io->C, io->R);
    if (io->P < 1 || io->N < 0) return fail(SDM_ESHAPE, "sdm_gds_step: P = %d, N = %d", io->P, io->N);
    if (ti < 0 || (ti + 1) * static_cast<int64_t>(io->P) > io->N)
        return fail(SDM_ESHAPE, "sdm_gds_step: step %lld needs (ti+1)*P <= N = %d", static_cast<long long>(ti), io->N);
    if (io->first_partial < 0 || io->first_partial > io->N || io->valid_last < 0 || io->valid_last > io->C)
        return fail(SDM_EINVAL, "sdm_gds_step: first_partial = %d, valid_last = %d", io->first_partial, io->valid_last);
    if (io->bank_dtype != SDM_F32 && io->bank_dtype != SDM_BF16)
        return fail(SDM_EINVAL, "sdm_gds_step: bank_dtype %d", io->bank_dtype);
    if (io->grad != nullptr && io->grad_dtype != SDM_F32 && io->grad_dtype != SDM_BF16)
        return fail(SDM_EINVAL, "sdm_gds_step: grad_dtype %d", io->grad_dtype);
    if (io->idx_bytes != 0 && io->idx_bytes != 4 && io->idx_bytes != 8)
        return fail(SDM_EINVAL, "sdm_gds_step: idx_bytes = %d (0 or 4: int32 ids; 8: int64 ids)", io->idx_bytes);
    if (io->val_bytes != 0 && io->val_bytes != 4 && io->val_bytes != 2)
        return fail(SDM_EINVAL, "sdm_gds_step: val_bytes = %d (0 or 4: float32 q_w; 2: bf16)", io->val_bytes);
    if (io->hd < 4 || io->hd > 4096 || io->hd % 4 != 0)
        return fail(SDM_ESHAPE, "sdm_gds_step: hd = %d (a multiple of 4 in 4..4096)", io->hd);
    if (io->rows < 1 || io->step_rows < 0 || io->gr_rows < 0) return fail(SDM_EINVAL, "sdm_gds_step: rows / step_rows / gr_rows");
    if (ti * io->step_rows + static_cast<int64_t>(io->P) * io->C > io->gr_rows)
        return fail(SDM_EINVAL, "sdm_gds_step: gr holds %lld rows, step %lld needs %lld", static_cast<long long>(io->gr_rows),
                    static_cast<long long>(ti), static_cast<long long>(ti * io->step_rows + static_cast<int64_t>(io->P) * io->C));
    if (io->bank == nullptr || io->q_idx == nullptr || io->q_w == nullptr || io->spay_q == nullptr || io->gr == nullptr)
        return fail(SDM_EINVAL, "sdm_gds_step: bank, q_idx, q_w, spay_q and gr are required");
    if (!aligned(io->bank, io->bank_dtype == SDM_BF16 ? 8 : 16) || !aligned(io->gr, 16) ||
        (io->grad != nullptr && !aligned(io->grad, io->grad_dtype == SDM_BF16 ? 8 : 16)))
        return fail(SDM_EALIGN, "sdm_gds_step: bank, gr and grad rows must be 16-byte aligned (8 for bf16)");
    if (!aligned(io->q_idx, io->idx_bytes == 8 ? 8 : 4) || !aligned(io->q_w, io->val_bytes == 2 ? 2 : 4) ||
        !aligned(io->spay_q, 4) || !aligned(io->d_q_w, 4))
        return fail(SDM_EALIGN, "sdm_gds_step: q_idx, q_w, spay_q or d_q_w misaligned");
    if (io->workspace != nullptr) {
        if (!aligned(io->workspace, 16)) return fail(SDM_EALIGN, "sdm_gds_step: workspace is not 16-byte aligned");
        const size_t need = sdm::gds_workspace_layout(io).total;
        if (io->workspace_bytes < need)
            return fail(SDM_EWORKSPACE, "sdm_gds_step: workspace needs %zu bytes, got %zu", need, io->workspace_bytes);
    }
    const hipError_t e = sdm::gds_launch(io, ti, st);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(SDM_EHIP, "sdm_gds_step: %s", hipGetErrorString(e));
    }
    return SDM_OK;
}

sdm_status sdm_gwr_step(const sdm_gwr_io* io, int64_t ti, hipStream_t st) {
    g_last_error.clear();
    if (io == nullptr) return fail(SDM_EINVAL, "sdm_gwr_step: io is NULL");
    if (io->C < 1 || io->C > 256 || io->W < 1 || io->W > 256)
        return fail(SDM_ESHAPE, "sdm_gwr_step: C = %d, W = %d outside 1..256", io->C, io->W);
    if (io->P < 1 || io->N < 0) return fail(SDM_ESHAPE, "sdm_gwr_step: P = %d, N = %d", io->P, io->N);
    if (ti < 0 || (ti + 1) * static_cast<int64_t>(io->P) > io->N)
        return fail(SDM_ESHAPE, "sdm_gwr_step: step %lld needs (ti+1)*P <= N = %d", static_cast<long long>(ti), io->N);
    if (io->first_partial < 0 || io->first_partial > io->N || io->valid_last < 0 || io->valid_last > io->C)
        return fail(SDM_EINVAL, "sdm_gwr_step: first_partial = %d, valid_last = %d", io->first_partial, io->valid_last);
    if (io->grad_dtype != SDM_F32 && io->grad_dtype != SDM_BF16)
        return fail(SDM_EINVAL, "sdm_gwr_step: grad_dtype %d", io->grad_dtype);
    if (io->idx_bytes != 0 && io->idx_bytes != 4 && io->idx_bytes != 8)
        return fail(SDM_EINVAL, "sdm_gwr_step: idx_bytes = %d (0 or 4: int32 ids; 8: int64 ids)", io->idx_bytes);
    if (io->hd < 4 || io->hd > 1024 || io->hd % 4 != 0)
        return fail(SDM_ESHAPE, "sdm_gwr_step: hd = %d (a multiple of 4 in 4..1024)", io->hd);
    if (io->rows < 1 || io->step_rows < 0 || io->dv_rows < 0) return fail(SDM_EINVAL, "sdm_gwr_step: rows / step_rows / dv_rows");
    if (ti * io->step_rows + static_cast<int64_t>(io->P) * io->C > io->dv_rows)
        return fail(SDM_EINVAL, "sdm_gwr_step: dv holds %lld rows, step %lld needs %lld", static_cast<long long>(io->dv_rows),
                    static_cast<long long>(ti), static_cast<long long>(ti * io->step_rows + static_cast<int64_t>(io->P) * io->C));
    if (io->grad == nullptr || io->k_idx == nullptr || io->w == nullptr || io->dv == nullptr)
        return fail(SDM_EINVAL, "sdm_gwr_step: grad, k_idx, w and dv are required");
    if (!aligned(io->grad, io->grad_dtype == SDM_BF16 ? 8 : 16) || !aligned(io->dv, 16) || !aligned(io->d_dv, 16))
        return fail(SDM_EALIGN, "sdm_gwr_step: grad, dv and d_dv rows must be 16-byte aligned (8 for bf16 grad)");
    if (!aligned(io->k_idx, io->idx_bytes == 8 ? 8 : 4) || !aligned(io->w, 4) || !aligned(io->d_k_pd, 4))
        return fail(SDM_EALIGN, "sdm_gwr_step: k_idx, w or d_k_pd misaligned");
    const hipError_t e = sdm::gwr_launch(io, ti, st);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(SDM_EHIP, "sdm_gwr_step: %s", hipGetErrorString(e));
    }
    return SDM_OK;
}

sdm_status sdm_pa_step(const sdm_pa_io* io, int64_t ti, hipStream_t st) {
    g_last_error.clear();
    if (io == nullptr) return fail(SDM_EINVAL, "sdm_pa_step: io is NULL");
    if (io->C < 1 || io->C > 256 || io->W < 1 || io->W > 256)
        return fail(SDM_ESHAPE, "sdm_pa_step: C = %d, W = %d outside 1..256", io->C, io->W);
    if (io->P < 1 || io->N < 0) return fail(SDM_ESHAPE, "sdm_pa_step: P = %d, N = %d", io->P, io->N);
    if (ti < 0 || (ti + 1) * static_cast<int64_t>(io->P) > io->N)
        return fail(SDM_ESHAPE, "sdm_pa_step: step %lld needs (ti+1)*P <= N = %d", static_cast<long long>(ti), io->N);
    if (io->grad_dtype != SDM_F32 && io->grad_dtype != SDM_BF16)
        return fail(SDM_EINVAL, "sdm_pa_step: grad_dtype %d", io->grad_dtype);
    if (io->bank_dtype != SDM_F32 && io->bank_dtype != SDM_BF16)
        return fail(SDM_EINVAL, "sdm_pa_step: bank_dtype %d", io->bank_dtype);
    if (io->val_bytes != 0 && io->val_bytes != 4 && io->val_bytes != 2)
        return fail(SDM_EINVAL, "sdm_pa_step: val_bytes = %d (0 or 4: float32 k_eff; 2: bf16)", io->val_bytes);
    if (io->hd < 4 || io->hd > 1024 || io->hd % 4 != 0)
        return fail(SDM_ESHAPE, "sdm_pa_step: hd = %d (a multiple of 4 in 4..1024)", io->hd);
    const int64_t pcw = static_cast<int64_t>(io->P) * io->C * io->W;
    if (io->rows < 1 || io->step_rows < 0 || io->dva_rows < 0 || io->snap_step_rows < 0)
        return fail(SDM_EINVAL, "sdm_pa_step: rows / step_rows / dva_rows / snap_step_rows");
    if (ti * io->step_rows + static_cast<int64_t>(io->P) * io->C > io->dva_rows)
        return fail(SDM_EINVAL, "sdm_pa_step: d_dva holds %lld rows, step %lld needs more", static_cast<long long>(io->dva_rows),
                    static_cast<long long>(ti));
    if (ti * io->snap_step_rows + pcw > io->snap_rows)
        return fail(SDM_EINVAL, "sdm_pa_step: snap holds %lld rows, step %lld needs %lld", static_cast<long long>(io->snap_rows),
                    static_cast<long long>(ti), static_cast<long long>(ti * io->snap_step_rows + pcw));
    if (io->grad == nullptr || io->snap == nullptr || io->krec == nullptr || io->k_eff == nullptr || io->beta == nullptr ||
        io->d_dva == nullptr)
        return fail(SDM_EINVAL, "sdm_pa_step: grad, snap, krec, k_eff, beta and d_dva are required");
    const uintptr_t ra = io->bank_dtype == SDM_BF16 ? 8 : 16;
    if (!aligned(io->grad, io->grad_dtype == SDM_BF16 ? 8 : 16) || !aligned(io->bank, ra) || !aligned(io->snap, ra) ||
        !aligned(io->d_dva, 16) || !aligned(io->krec, 16))
        return fail(SDM_EALIGN, "sdm_pa_step: grad, bank, snap, d_dva or krec misaligned");
    if (!aligned(io->k_eff, io->val_bytes == 2 ? 2 : 4) || !aligned(io->beta, 4) || !aligned(io->g_decay, 4) ||
        !aligned(io->d_k_eff, 4))
        return fail(SDM_EALIGN, "sdm_pa_step: k_eff, beta, g_decay or d_k_eff misaligned");
    if (io->workspace != nullptr) {
        if (!aligned(io->workspace, 16)) return fail(SDM_EALIGN, "sdm_pa_step: workspace is not 16-byte aligned");
        const size_t need = sdm::pa_workspace_layout(io).total;
        if (io->workspace_bytes < need)
            return fail(SDM_EWORKSPACE, "sdm_pa_step: workspace needs %zu bytes, got %zu", need, io->workspace_bytes);
    }
    const hipError_t e = sdm::pa_launch(io, ti, st);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(SDM_EHIP, "sdm_pa_step: %s", hipGetErrorString(e));
    }
    return SDM_OK;
}

sdm_status sdm_dw_step(const sdm_dw_io* io, int64_t ti, hipStream_t st) {
    g_last_error.clear();
    if (io == nullptr) return fail(SDM_EINVAL, "sdm_dw_step: io is NULL");
    const sdm_status rc = check_dw_io(io, ti, "sdm_dw_step");
    if (rc != SDM_OK) return rc;
    sdm::DwLaunch L;
    L.io = io;
    L.ti = ti;
    const hipError_t e = sdm::dw_launch(L, st);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(SDM_EHIP, "sdm_dw_step: %s", hipGetErrorString(e));
    }
    return SDM_OK;
}

sdm_status sdm_dw_step_noalloc(const sdm_dw_io* io, int64_t ti, hipStream_t st) {
    g_last_error.clear();
    if (io == nullptr) return fail(SDM_EINVAL, "sdm_dw_step_noalloc: io is NULL");
    if (io->workspace != nullptr)
        return fail(SDM_EINVAL, "sdm_dw_step_noalloc: workspace must be NULL (the library's fixed device array is used)");
    const sdm_status rc = check_dw_io(io, ti, "sdm_dw_step_noalloc");
    if (rc != SDM_OK) return rc;
    size_t need = 0, cap = 0;
    if (!sdm::dw_static_fits(io, &need, &cap))
        return fail(SDM_EWORKSPACE,
                    "sdm_dw_step_noalloc: P*C*W = %lld positions and %zu bytes of partial rows exceed the fixed array "
                    "(at most 4194304 positions and %zu bytes); use sdm_dw_step with a workspace",
                    static_cast<long long>(static_cast<int64_t>(io->P) * io->C * io->W), need, cap);
    hipError_t e = device_setup(nullptr);
    if (e == hipSuccess) e = sdm::dw_static_setup();
    if (e != hipSuccess) return fail(SDM_EHIP, "sdm_dw_step_noalloc: set-up: %s", hipGetErrorString(e));
    sdm::DwLaunch L;
    L.io = io;
    L.ti = ti;
    e = sdm::dw_launch_static(L, st);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(SDM_EHIP, "sdm_dw_step_noalloc: %s", hipGetErrorString(e));
    }
    return SDM_OK;
}

}  // extern "C"
