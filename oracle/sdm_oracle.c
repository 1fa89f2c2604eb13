/*
 * Plain, slow CPU oracle for the forward hot path of the chunked sparse-delta-memory (SDM)
 * recurrence: Phase 1 (sort by slot, segmented log-cumsums, flags, positions, kind rows,
 * mover records, tile bounds, pair sums A / QK) and the DW decay-and-write step.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path links or calls this file; only the
 * tests, the smoke check and the benchmark's CPU-baseline leg do. It shares no code, header,
 * table or helper with the HIP implementation.
 *
 * Source of every definition: the page "sparse_delta_memory/cuda/phase1_cuda.py"
 * (module docstring: the quantity list log_k, log_q, rex, cpe, is_last/is_only, k_eff, q_w,
 * a, qk, pos_k/pos_q, q_last/q_only; the Outputs / Records comments; p1_keys_zw_kernel for
 * keys and payloads; p1_scan_kernel for groups, gate contributions, packed positions and
 * sorted kind rows; p1_pairs_kernel comment for the pair terms) and the pages
 * "sparse_delta_memory/cuda/mover_da2_cuda.py" (module docstring: the DW definition) and
 * "sparse_delta_memory/cuda/mover_fx_cuda.py" (module docstring: the DW bit contract).
 *
 * Arithmetic is double precision; every result is produced from its definition with no
 * blocking, fusion or reordering beyond the plain loops below. Floating outputs are returned
 * in double (the caller rounds once to float32 where it compares).
 *
 * Readings taken where the pages leave a step open (each listed in the design notes):
 *  - payload word: lane in bits 0-7, read (Q) flag bit 8, token bits 9-16, invalid bit 17;
 *  - invalid entries (tokens at or past the chunk's valid count) sort after all valid
 *    entries in entry order and each forms a group of its own;
 *  - a K entry contributes its token's gate once per (token, slot): a K entry whose
 *    predecessor in the group is a K entry of the same token contributes 0 (a "repeat");
 *  - gates are per token, or per (token, K lane) as the scan kernel's width / lane-stride
 *    addressing allows; with per-lane gates the token's lowest lane writing the slot applies.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_FIRST 0x80000000u
#define OR_LAST 0x40000000u
#define OR_INVALID 0x20000u
#define OR_ISQ 0x100u
#define OR_TOKEN_SHIFT 9
#define OR_DIST_SHIFT 18
#define OR_DIST_MAX 4095u
#define OR_POS_AFTER_SHIFT 17
#define OR_POS_SIZE_SHIFT 24
#define OR_POS_COUNT_MAX 127u

/* One chunk's inputs (pointers already offset to the chunk). */
typedef struct {
    int C, W, R;
    int t_valid;        /* tokens t < t_valid are valid */
    int64_t id_base;    /* (chunk mod P) * stream_offset: local slot = id - id_base */
    const int32_t* k_idx;   /* [C, W] absolute slot ids */
    const int32_t* q_idx;   /* [C, R] */
    const float* k_val;     /* [C, W] */
    const float* q_val;     /* [C, R] */
    const float* g;         /* gates (log decays, <= 0): g[t * g_width + lane * g_lane_stride] is the
                               gate of token t's K lane `lane` ([C] per token: width 1, stride 0;
                               [C, W] per token and lane: width W, stride 1) */
    int tile_len;           /* L of tiles_k */
    int g_width;
    int g_lane_stride;
    int val_bf16;           /* 1: the values are bfloat16 (k_val / q_val hold their exact float
                               values); cpe, k_eff, q_w and the records' cpe are then bfloat16 too
                               (each the exact value rounded once, to nearest even), and the DW step
                               scales the base row by that rounded cpe (page
                               "sparse_delta_memory/cuda/phase1_cuda.py": the value type of the
                               Outputs struct, and the mover record comment "cpe as the ValT value
                               widened") */
} oracle_chunk_in;

/* x rounded to the nearest bfloat16 value (8 significant bits, float's exponent range), ties to
 * even: x = m 2^e with 0.5 <= |m| < 1 has the quantum 2^(e - 8) in the normal range and 2^-133
 * below it; nearbyint rounds to the nearest integer, ties to even, in the default rounding mode.
 * Finite inputs only (the values here are far from bfloat16's overflow). */
double oracle_round_bf16(double x) {
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    (void)frexp(x, &e);
    const int qe = (e > -125 ? e : -125) - 8;
    return ldexp(nearbyint(ldexp(x, -qe)), qe);
}

static double oracle_val_round(const oracle_chunk_in* in, double x) {
    return in->val_bf16 ? oracle_round_bf16(x) : x;
}

/* One chunk's outputs; any pointer may be NULL to skip that field. */
typedef struct {
    double* log_k;      /* [C, W] */
    double* rex;        /* [C, W] */
    double* cpe;        /* [C, W] */
    double* k_eff;      /* [C, W] */
    int8_t* is_last;    /* [C, W] */
    int8_t* is_only;    /* [C, W] */
    int32_t* pos_k;     /* [C, W] */
    double* log_q;      /* [C, R] */
    double* q_w;        /* [C, R] */
    int32_t* pos_q;     /* [C, R] */
    int8_t* q_last;     /* [C, R] */
    int8_t* q_only;     /* [C, R] */
    int32_t* spay_k;    /* [C*W] sorted K-only row elements */
    int32_t* spay_q;    /* [C*R] sorted Q-only row elements */
    int32_t* krec_slot; /* [C*W] absolute slot (0 for padding) */
    double* krec_sc;    /* [C*W] k * exp(rex) (0 for padding) */
    double* krec_cpe;   /* [C*W] cpe (1 for padding) */
    int32_t* tiles_k;   /* [ceil(C*W/L) + 1] */
    double* a;          /* [C, C] */
    double* qk;         /* [C, C] */
    int32_t* perm;      /* [C*(W+R)] entry index r at sorted position rho */
    int64_t* repeats;   /* [1] repeated K entries of the chunk */
    double* a_mag;      /* [C, C] sum of |term| per cell of A (the float evaluation error scale) */
    double* qk_mag;     /* [C, C] the same for QK */
    int32_t* a_cnt;     /* [C, C] number of terms per cell of A */
    int32_t* qk_cnt;    /* [C, C] the same for QK */
    int32_t* gord_k;    /* [C*W] per K-row position: the ordinal of its group among the chunk's groups with
                           a valid K entry, in K-row (slot) order; -1 for padding (the dense group
                           ordinal of the compact rows, page "sparse_delta_memory/cuda/mover_fx_cuda.py",
                           module docstring and the WR walk) */
} oracle_chunk_out;

typedef struct {
    int64_t key;
    int32_t r;
    int32_t invalid;
} oracle_ent;

/* Sort order of the chunk: valid entries by (local slot, entry index), then invalid entries
 * by entry index alone. The entry index is unique, so this is a total order (no ties). */
static int oracle_cmp(const void* pa, const void* pb) {
    const oracle_ent* a = (const oracle_ent*)pa;
    const oracle_ent* b = (const oracle_ent*)pb;
    if (a->invalid != b->invalid) return a->invalid < b->invalid ? -1 : 1;
    /* Invalid entries all take the largest key, so among themselves only r orders them. */
    if (!a->invalid && a->key != b->key) return a->key < b->key ? -1 : 1;
    if (a->r != b->r) return a->r < b->r ? -1 : 1;
    return 0;
}

/* Per-entry facts of the sorted row, filled by oracle_build. */
typedef struct {
    int n;
    oracle_ent* ent;     /* [n] sorted */
    int* tok;            /* [n] token of sorted entry */
    int* lane;           /* [n] lane within its kind */
    int* isq;            /* [n] 1 for a read entry */
    int* gstart;         /* [n] sorted position of the entry's group head */
    int* gend;           /* [n] one past the group's last sorted position */
    double* x;           /* [n] gate contribution */
    double* L;           /* [n] inclusive log-cumsum inside the group */
    double* rexv;        /* [n] sum of x after the entry inside the group */
    int* kb;             /* [n] valid K entries before, in the group */
    int* ka;             /* [n] valid K entries after */
    int* qb;             /* [n] valid Q entries before */
    int* qa;             /* [n] valid Q entries after */
    int64_t repeats;
} oracle_row;

static void oracle_row_free(oracle_row* w) {
    free(w->ent); free(w->tok); free(w->lane); free(w->isq); free(w->gstart); free(w->gend);
    free(w->x); free(w->L); free(w->rexv); free(w->kb); free(w->ka); free(w->qb); free(w->qa);
}

static int oracle_build(const oracle_chunk_in* in, oracle_row* w) {
    const int wr = in->W + in->R;
    const int n = in->C * wr;
    memset(w, 0, sizeof(*w));
    w->n = n;
    w->ent = (oracle_ent*)malloc(sizeof(oracle_ent) * (size_t)(n > 0 ? n : 1));
    w->tok = (int*)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
    w->lane = (int*)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
    w->isq = (int*)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
    w->gstart = (int*)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
    w->gend = (int*)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
    w->x = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    w->L = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    w->rexv = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    w->kb = (int*)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
    w->ka = (int*)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
    w->qb = (int*)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
    w->qa = (int*)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
    if (!w->ent || !w->tok || !w->lane || !w->isq || !w->gstart || !w->gend || !w->x || !w->L ||
        !w->rexv || !w->kb || !w->ka || !w->qb || !w->qa) {
        oracle_row_free(w);
        return -1;
    }
    /* Entries: r = t (W + R) + j, K lanes j < W first, then the R read lanes. */
    for (int r = 0; r < n; ++r) {
        const int t = r / wr, j = r % wr;
        const int q = j >= in->W;
        const int lane = q ? j - in->W : j;
        const int64_t id = q ? (int64_t)in->q_idx[t * in->R + lane] : (int64_t)in->k_idx[t * in->W + lane];
        w->ent[r].key = id - in->id_base;
        w->ent[r].r = r;
        w->ent[r].invalid = t >= in->t_valid;
    }
    qsort(w->ent, (size_t)n, sizeof(oracle_ent), oracle_cmp);
    for (int p = 0; p < n; ++p) {
        const int r = w->ent[p].r;
        const int j = r % wr;
        w->tok[p] = r / wr;
        w->isq[p] = j >= in->W;
        w->lane[p] = w->isq[p] ? j - in->W : j;
    }
    /* Groups: maximal runs of valid entries with one slot; an invalid entry is its own group. */
    for (int p = 0; p < n;) {
        int e = p + 1;
        if (!w->ent[p].invalid) {
            while (e < n && !w->ent[e].invalid && w->ent[e].key == w->ent[p].key) ++e;
        }
        for (int u = p; u < e; ++u) {
            w->gstart[u] = p;
            w->gend[u] = e;
        }
        p = e;
    }
    /* Gate contributions: a valid K entry adds its gate unless the previous entry of its group is
     * a K entry of the same token. A token's writes to one slot are adjacent in the group and in
     * lane order, so the gate applied is that of the token's lowest lane writing the slot. */
    w->repeats = 0;
    for (int p = 0; p < n; ++p) {
        w->x[p] = 0.0;
        if (w->ent[p].invalid || w->isq[p]) continue;
        const int rep = p > w->gstart[p] && !w->isq[p - 1] && w->tok[p - 1] == w->tok[p];
        if (rep) {
            ++w->repeats;
        } else {
            w->x[p] = (double)in->g[w->tok[p] * in->g_width + w->lane[p] * in->g_lane_stride];
        }
    }
    /* Inclusive log-cumsum, sum after, and the peers of each kind before / after. */
    for (int p = 0; p < n; ++p) {
        const int s = w->gstart[p], e = w->gend[p];
        double L = 0.0, after = 0.0;
        int kb = 0, ka = 0, qb = 0, qa = 0;
        for (int u = s; u <= p; ++u) L += w->x[u];
        for (int u = p + 1; u < e; ++u) after += w->x[u];
        for (int u = s; u < p; ++u) {
            if (w->ent[u].invalid) continue;
            if (w->isq[u]) ++qb; else ++kb;
        }
        for (int u = p + 1; u < e; ++u) {
            if (w->ent[u].invalid) continue;
            if (w->isq[u]) ++qa; else ++ka;
        }
        w->L[p] = L;
        w->rexv[p] = after;
        w->kb[p] = kb;
        w->ka[p] = ka;
        w->qb[p] = qb;
        w->qa[p] = qa;
    }
    return 0;
}

static uint32_t oracle_umin(uint32_t a, uint32_t b) { return a < b ? a : b; }

/* Phase 1 of one chunk. Returns 0, or -1 when memory runs out. */
int oracle_phase1_chunk(const oracle_chunk_in* in, const oracle_chunk_out* out) {
    oracle_row w;
    if (oracle_build(in, &w) != 0) return -1;
    const int C = in->C, W = in->W, R = in->R;
    const int n = w.n;
    const int nk = C * W;
    int jk = 0, jq = 0;
    int kgroups = 0;   /* groups with a valid K entry so far */
    for (int p = 0; p < n; ++p) {
        const int t = w.tok[p], lane = w.lane[p], q = w.isq[p];
        const int valid = !w.ent[p].invalid;
        const uint32_t r = (uint32_t)w.ent[p].r;
        const uint32_t payload = (uint32_t)lane | (q ? OR_ISQ : 0u) | ((uint32_t)t << OR_TOKEN_SHIFT) |
                                 (valid ? 0u : OR_INVALID);
        const int before = q ? w.qb[p] : w.kb[p];
        const int after = q ? w.qa[p] : w.ka[p];
        (void)r;
        /* Packed position: sorted position, peers after (saturating), peers in group. */
        uint32_t packed = (uint32_t)p;
        if (valid) {
            packed |= oracle_umin((uint32_t)after, OR_POS_COUNT_MAX) << OR_POS_AFTER_SHIFT;
            packed |= oracle_umin((uint32_t)(before + 1 + after), OR_POS_COUNT_MAX) << OR_POS_SIZE_SHIFT;
        }
        /* Element of the sorted kind row. */
        uint32_t sorted;
        if (valid) {
            sorted = (payload & 0x3FFFFu) | oracle_umin((uint32_t)before, OR_DIST_MAX) << OR_DIST_SHIFT |
                     (before == 0 ? OR_FIRST : 0u) | (after == 0 ? OR_LAST : 0u);
        } else {
            sorted = payload | OR_FIRST | OR_LAST;
        }
        const double L = valid ? w.L[p] : 0.0;
        const double v = valid ? (double)(q ? in->q_val[t * R + lane] : in->k_val[t * W + lane]) : 0.0;
        if (out->perm) out->perm[p] = (int32_t)w.ent[p].r;
        if (q) {
            const int o = t * R + lane;
            if (out->log_q) out->log_q[o] = L;
            if (out->q_w) out->q_w[o] = valid ? oracle_val_round(in, v * exp(L)) : 0.0;
            if (out->pos_q) out->pos_q[o] = (int32_t)packed;
            if (out->q_last) out->q_last[o] = (int8_t)(valid && after == 0);
            if (out->q_only) out->q_only[o] = (int8_t)(valid && after == 0 && before == 0);
            if (out->spay_q) out->spay_q[jq] = (int32_t)sorted;
            ++jq;
        } else {
            const int o = t * W + lane;
            const double rexv = valid ? w.rexv[p] : 0.0;
            const double cpe = valid ? oracle_val_round(in, exp(L + rexv)) : 1.0;
            if (out->log_k) out->log_k[o] = L;
            if (out->rex) out->rex[o] = rexv;
            if (out->cpe) out->cpe[o] = cpe;
            if (out->k_eff) out->k_eff[o] = valid ? oracle_val_round(in, v * exp(L)) : 0.0;
            if (out->is_last) out->is_last[o] = (int8_t)(valid && after == 0);
            if (out->is_only) out->is_only[o] = (int8_t)(valid && after == 0 && before == 0);
            if (out->pos_k) out->pos_k[o] = (int32_t)packed;
            if (out->spay_k) out->spay_k[jk] = (int32_t)sorted;
            if (out->krec_slot) out->krec_slot[jk] = valid ? (int32_t)(w.ent[p].key + in->id_base) : 0;
            if (out->krec_sc) out->krec_sc[jk] = valid ? v * exp(rexv) : 0.0;
            if (out->krec_cpe) out->krec_cpe[jk] = valid ? cpe : 1.0;
            if (valid && before == 0) ++kgroups;   /* the group's first valid K entry */
            if (out->gord_k) out->gord_k[jk] = valid ? kgroups - 1 : -1;
            ++jk;
        }
    }
    /* Tile bounds of the K-only row: the first index >= t L holding a FIRST (nk if none),
     * then nk. FIRST is bit 31 of the kind-row element. */
    if (out->tiles_k) {
        if (out->spay_k == NULL) {
            oracle_row_free(&w);
            return -2;
        }
        const int L = in->tile_len > 0 ? in->tile_len : 1;
        const int ntk = (nk + L - 1) / L;
        for (int t = 0; t < ntk; ++t) {
            int j = t * L;
            while (j < nk && !((uint32_t)out->spay_k[j] & OR_FIRST)) ++j;
            out->tiles_k[t] = j;
        }
        out->tiles_k[ntk] = nk;
    }
    /* Pair sums: every valid entry e with an earlier valid K entry f of its group adds
     * val_e * val_f * exp(L_e - L_f) to cell (token(e), token(f)) of A (e a K entry of another
     * token) or QK (e a Q entry). */
    if (out->a) memset(out->a, 0, sizeof(double) * (size_t)C * (size_t)C);
    if (out->qk) memset(out->qk, 0, sizeof(double) * (size_t)C * (size_t)C);
    if (out->a_mag) memset(out->a_mag, 0, sizeof(double) * (size_t)C * (size_t)C);
    if (out->qk_mag) memset(out->qk_mag, 0, sizeof(double) * (size_t)C * (size_t)C);
    if (out->a_cnt) memset(out->a_cnt, 0, sizeof(int32_t) * (size_t)C * (size_t)C);
    if (out->qk_cnt) memset(out->qk_cnt, 0, sizeof(int32_t) * (size_t)C * (size_t)C);
    if (out->a || out->qk || out->a_mag || out->qk_mag || out->a_cnt || out->qk_cnt) {
        for (int p = 0; p < n; ++p) {
            if (w.ent[p].invalid) continue;
            const int ti = w.tok[p];
            const int q = w.isq[p];
            const double ve = q ? (double)in->q_val[ti * R + w.lane[p]] : (double)in->k_val[ti * W + w.lane[p]];
            for (int u = w.gstart[p]; u < p; ++u) {
                if (w.isq[u]) continue; /* only K entries are written */
                const int tj = w.tok[u];
                const double vf = (double)in->k_val[tj * W + w.lane[u]];
                const double term = ve * vf * exp(w.L[p] - w.L[u]);
                if (q) {
                    if (out->qk) out->qk[ti * C + tj] += term;
                    if (out->qk_mag) out->qk_mag[ti * C + tj] += fabs(term);
                    if (out->qk_cnt) out->qk_cnt[ti * C + tj] += 1;
                } else if (tj != ti) {
                    if (out->a) out->a[ti * C + tj] += term;
                    if (out->a_mag) out->a_mag[ti * C + tj] += fabs(term);
                    if (out->a_cnt) out->a_cnt[ti * C + tj] += 1;
                }
            }
        }
    }
    if (out->repeats) out->repeats[0] = w.repeats;
    oracle_row_free(&w);
    return 0;
}

/* Slots of the chunk's valid K groups (ascending local slot, so ascending absolute slot).
 * Writes them to slots (when not NULL) and returns their count, or -1. */
int64_t oracle_dw_slots(const oracle_chunk_in* in, int64_t* slots) {
    oracle_row w;
    if (oracle_build(in, &w) != 0) return -1;
    int64_t cnt = 0;
    for (int p = 0; p < w.n; ++p) {
        if (w.ent[p].invalid || w.isq[p] || w.kb[p] != 0) continue; /* first valid K of its group */
        if (slots) slots[cnt] = w.ent[p].key + in->id_base;
        ++cnt;
    }
    oracle_row_free(&w);
    return cnt;
}

/* The DW step of one chunk: for every valid K group (slot s, ascending),
 *   new[s] = base[s] * exp(G_s) + sum over its valid K entries m of k_m exp(rex_m) dv[token(m)],
 * G_s the total gate of the group. base / out hold one row of hd values per group, in the order
 * oracle_dw_slots returns; dv holds the chunk's C token rows. When mag is not NULL it receives,
 * per element, |base exp(G)| + sum |k exp(rex) dv|, the magnitude that bounds the rounding
 * error of any float evaluation. Returns the group count, or -1. */
int64_t oracle_dw_apply(const oracle_chunk_in* in, int hd, const double* dv, const double* base, double* out,
                        double* mag) {
    oracle_row w;
    if (oracle_build(in, &w) != 0) return -1;
    int64_t gi = -1;
    for (int p = 0; p < w.n; ++p) {
        if (w.ent[p].invalid || w.isq[p]) continue;
        if (w.kb[p] == 0) {
            ++gi;
            /* exp of the group's total gate: L at this entry plus the sum after it (rounded to
             * bfloat16 with bfloat16 values, as the records carry it). */
            const double cpe = oracle_val_round(in, exp(w.L[p] + w.rexv[p]));
            for (int d = 0; d < hd; ++d) {
                out[gi * hd + d] = base[gi * hd + d] * cpe;
                if (mag) mag[gi * hd + d] = fabs(base[gi * hd + d] * cpe);
            }
        }
        const double sc = (double)in->k_val[w.tok[p] * in->W + w.lane[p]] * exp(w.rexv[p]);
        for (int d = 0; d < hd; ++d) {
            const double term = sc * dv[(int64_t)w.tok[p] * hd + d];
            out[gi * hd + d] += term;
            if (mag) mag[gi * hd + d] += fabs(term);
        }
    }
    oracle_row_free(&w);
    return gi + 1;
}
