// Host-only entry points over the same plan and slot-pool code that the HIP
// library links, so the profile validation and the slot state machine can
// be exercised on a machine without a GPU.  Built with the host compiler
// into libfd_host.so; never linked into the product library.
#include <new>
#include <string>

#include "../../include/fd.h"
#include "fd_plan.h"
#include "slot_pool.h"

namespace {
thread_local std::string g_err;
}

extern "C" {

fd_status fdh_plan(const fd_config* cfg, fd_sizes* out) {
    if (!cfg || !out) return FD_E_INVAL;
    fd::Plan p;
    fd_status st = fd::make_plan(*cfg, &p, &g_err);
    if (st != FD_OK) return st;
    out->packed_weights = p.packed_bytes;
    out->kv_arena = p.kv_bytes_total;
    out->workspace = p.workspace_bytes;
    out->slot_table = p.slot_table_bytes;
    return FD_OK;
}

const char* fdh_last_error(void) { return g_err.c_str(); }

// Tiling chosen for one projection: out[0..8] = NB, KB, R, P, MG, MTG, n_groups, grid, KT.
void fdh_gemm_shape(int N, int K, int wt, int MT, int32_t* out) {
    fd::GemmShape g = fd::choose_gemm(N, K, wt ? 32 : 16, MT, 256);
    out[0] = g.NB; out[1] = g.KB; out[2] = g.R; out[3] = g.P; out[4] = g.MG; out[5] = g.MTG;
    out[6] = g.n_groups; out[7] = g.grid(); out[8] = g.KT;
}

// Tiling of the projections as the plan of cfg chose it (FD_TUNE applies):
// out[4*i + 0..3] = R, P, k-halves, grid for i = QKV, O, gate/up, down of
// the main stack, then (i = 4..7) of the depth stack (zeros without one).
fd_status fdh_stack_shapes(const fd_config* cfg, int32_t* out) {
    if (!cfg || !out) return FD_E_INVAL;
    fd::Plan p;
    fd_status st = fd::make_plan(*cfg, &p, &g_err);
    if (st != FD_OK) return st;
    const fd::GemmShape* g[8] = {&p.main.qkv, &p.main.o, &p.main.gu, &p.main.down,
                                 &p.dstack.qkv, &p.dstack.o, &p.dstack.gu, &p.dstack.down};
    for (int i = 0; i < 8; ++i) {
        const bool have = i < 4 || p.depth;
        out[4 * i + 0] = have ? g[i]->R : 0;
        out[4 * i + 1] = have ? g[i]->P : 0;
        out[4 * i + 2] = have ? g[i]->kh : 0;
        out[4 * i + 3] = have ? g[i]->grid() : 0;
    }
    return FD_OK;
}

// Row tiling as the plan of cfg chose it: out[0] = padded 16-row tiles;
// out[1 + 2*i], out[2 + 2*i] = m-groups and tiles per m-group of QKV, O,
// gate/up, down and (with a vocabulary) the output head.
fd_status fdh_stack_mtiles(const fd_config* cfg, int32_t* out) {
    if (!cfg || !out) return FD_E_INVAL;
    fd::Plan p;
    fd_status st = fd::make_plan(*cfg, &p, &g_err);
    if (st != FD_OK) return st;
    out[0] = p.MT;
    const fd::GemmShape* g[5] = {&p.main.qkv, &p.main.o, &p.main.gu, &p.main.down, &p.hshape};
    for (int i = 0; i < 5; ++i) {
        out[1 + 2 * i] = g[i]->MG;
        out[2 + 2 * i] = g[i]->MTG;
    }
    return FD_OK;
}

void* fdh_pool_new(int n_slots, int max_context, int rolling) {
    return new (std::nothrow) fd::SlotPool(n_slots, max_context, rolling != 0);
}
void fdh_pool_delete(void* p) { delete (fd::SlotPool*)p; }
fd_status fdh_pool_alloc(void* p, int32_t n, int32_t* out) { return ((fd::SlotPool*)p)->alloc(n, out); }
fd_status fdh_pool_free(void* p, const int32_t* ids, int32_t n) { return ((fd::SlotPool*)p)->free(ids, n); }
fd_status fdh_pool_set_position(void* p, int32_t s, int32_t pos) {
    return ((fd::SlotPool*)p)->set_position(s, pos);
}
fd_status fdh_pool_state(void* p, int32_t s, int32_t* a, int32_t* pos) {
    return ((fd::SlotPool*)p)->state(s, a, pos);
}
int fdh_pool_any_full(void* p) {
    int w = -1;
    return ((fd::SlotPool*)p)->any_full(&w) ? w : -1;
}
void fdh_pool_advance(void* p) { ((fd::SlotPool*)p)->advance(); }
int fdh_pool_dirty(void* p) { return ((fd::SlotPool*)p)->dirty() ? 1 : 0; }
void fdh_pool_clear_dirty(void* p) { ((fd::SlotPool*)p)->clear_dirty(); }
void fdh_pool_image(void* p, int32_t* dst) { ((fd::SlotPool*)p)->image(dst); }
void fdh_pool_mark_stale(void* p) { ((fd::SlotPool*)p)->mark_stale(); }
int fdh_pool_any_stale(void* p) {
    int w = -1;
    return ((fd::SlotPool*)p)->any_stale(&w) ? w : -1;
}

}  // extern "C"
