// C ABI of the decode step: profile validation, weight packing, the slot
// table, and the per-frame launch sequence.  Declarations and contracts are
// in include/fd.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/fd.h"
#include "fd_internal.h"
#include "fd_kernels.h"
#include "fd_plan.h"
#include "slot_pool.h"

namespace {

thread_local std::string g_global_err;

constexpr int kRing = 4;

}  // namespace

struct fd_ctx {
    fd::Plan plan;
    fd::SlotPool slots;
    fd_buffers buf{};
    // workspace the step's kernels use: buf.workspace, or the library's
    // static scratch during fd_step_static
    uint8_t* ws = nullptr;
    bool no_timing = false;  // fd_step_static: never create events
    int device = 0;
    std::string err;
    int32_t* pinned[kRing] = {};
    hipEvent_t ev[kRing] = {};
    bool ev_used[kRing] = {};
    int ring = 0;
    // per-kernel timing
    bool prof = false;
    std::vector<hipEvent_t> ev_pool;
    std::vector<std::pair<int, std::pair<hipEvent_t, hipEvent_t>>> prof_pending;
    double prof_ms[FD_N_KINDS] = {};
    int64_t prof_n[FD_N_KINDS] = {};
    // persistent walk of the whole step (built at init for FD_EXEC_WALK)
    fd::WalkArgs walk{};
    fd::WalkShape walk_shape{};
    int walk_grid = 0;
    // input rows of the output head (written by the step's final norm)
    const void* head_x = nullptr;
    const void* head_x_lo = nullptr;
    bool walk_launched = false;
    bool walk_abort_next = false;  // fd_walk_abort_next: the next walk starts aborted
    // device-clock trace of one layer's attention launch (fd_trace_attention)
    uint64_t* trace = nullptr;
    int trace_layer = -1;
    explicit fd_ctx(const fd::Plan& p) : plan(p), slots(p.S, p.cfg.max_context, p.ring) {}
};

namespace {

fd_status fail(fd_ctx* c, fd_status st, const std::string& msg) {
    if (c) c->err = msg;
    else g_global_err = msg;
    return st;
}

fd_status hip_fail(fd_ctx* c, hipError_t e, const char* where) {
    return fail(c, FD_E_DEVICE, std::string(where) + ": " + hipGetErrorString(e));
}

bool aligned(const void* p) { return p && ((uintptr_t)p % fd::kAlign) == 0; }

uint8_t* P(const fd_ctx* c, uint64_t off) { return (uint8_t*)c->buf.packed_weights + off; }
uint8_t* Wk(const fd_ctx* c, uint64_t off) { return c->ws + off; }

// FP8 or fp16 weight codes: the per-row scales stored after a matrix's
// tiles (else null)
const float* wscale(const fd_ctx* c, uint64_t off, const fd::GemmShape& g) {
    return c->plan.wkind >= 2 ? (const float*)(P(c, off) + (size_t)g.NB * g.KB * fd::kTileBytes) : nullptr;
}

int32_t* slot_active(const fd_ctx* c) { return (int32_t*)c->buf.slot_table; }
int32_t* slot_pos(const fd_ctx* c) { return (int32_t*)c->buf.slot_table + c->plan.S; }
int32_t* slot_order(const fd_ctx* c) { return (int32_t*)c->buf.slot_table + 2 * c->plan.S; }

fd_status check_layer(const fd_layer_weights& lw) {
    if (!lw.wq || !lw.wk || !lw.wv || !lw.wo || !lw.w_gate || !lw.w_up || !lw.w_down ||
        !lw.g_attn || !lw.g_ffn)
        return FD_E_INVAL;
    return FD_OK;
}

// wt: weight format (0 fp32, 1 bf16, 2 FP8 or 3 fp16 codes of bf16 sources,
// whose per-row scales go right after the tiles)
hipError_t pack(const fd::GemmShape& g, int wt, const void* s0, int r0, const void* s1, int r1,
                const void* s2, int interleave, uint8_t* dst, hipStream_t st) {
    fd::PackArgs a{};
    a.src[0] = s0;
    a.src[1] = s1;
    a.src[2] = s2;
    a.rows[0] = r0;
    a.rows[1] = r1;
    a.rows[2] = 0;
    a.interleave = interleave;
    a.N = g.N;
    a.K = g.K;
    a.KB = g.KB;
    a.dst = dst;
    a.scale = wt >= 2 ? (float*)(dst + (size_t)g.NB * g.KB * fd::kTileBytes) : nullptr;
    a.f16 = wt == 3;
    a.x3 = g.x3;
    return fd::launch_pack(a, wt, st);
}

hipError_t pack_stack(fd_ctx* c, const fd::StackPlan& sp, const fd_layer_weights* lw,
                      const float* g_final, hipStream_t st) {
    const fd::StackDims& d = sp.dims;
    const int wt = c->plan.wkind;
    hipError_t e = hipSuccess;
    for (int l = 0; l < d.L && e == hipSuccess; ++l) {
        const fd::LayerOffsets& lo = sp.layers[l];
        e = pack(sp.qkv, wt, lw[l].wq, d.hq * d.hd, lw[l].wk, d.hkv * d.hd, lw[l].wv, 0,
                 P(c, lo.qkv), st);
        if (e == hipSuccess) e = pack(sp.o, wt, lw[l].wo, d.d, nullptr, 0, nullptr, 0, P(c, lo.o), st);
        if (e == hipSuccess)
            e = pack(sp.gu, wt, lw[l].w_gate, 0, lw[l].w_up, 0, nullptr, 1, P(c, lo.gu), st);
        if (e == hipSuccess)
            e = pack(sp.down, wt, lw[l].w_down, d.d, nullptr, 0, nullptr, 0, P(c, lo.down), st);
        if (e == hipSuccess)
            e = hipMemcpyAsync(P(c, lo.g_attn), lw[l].g_attn, 4ull * d.d, hipMemcpyDeviceToDevice, st);
        if (e == hipSuccess)
            e = hipMemcpyAsync(P(c, lo.g_ffn), lw[l].g_ffn, 4ull * d.d, hipMemcpyDeviceToDevice, st);
    }
    if (e == hipSuccess)
        e = hipMemcpyAsync(P(c, sp.g_final), g_final, 4ull * d.d, hipMemcpyDeviceToDevice, st);
    return e;
}

// Constant tables of one stack: rotary cos/sin (double -> fp32), and the
// per-(layer, kv head) scale factors used by the append and the softmax.
hipError_t upload_tables(fd_ctx* c, const fd::StackPlan& sp, const std::vector<float>& sig,
                         bool fp8, hipStream_t st) {
    const fd::StackDims& d = sp.dims;
    const int Lm = std::max(d.L, 1);
    std::vector<float> rope((size_t)d.T * d.hd);
    for (int p = 0; p < d.T; ++p)
        for (int i = 0; i < d.hd / 2; ++i) {
            const double theta = std::pow((double)c->plan.cfg.rope_base, -2.0 * i / d.hd);
            const double ang = (double)p * theta;
            rope[((size_t)p * (d.hd / 2) + i) * 2 + 0] = (float)std::cos(ang);
            rope[((size_t)p * (d.hd / 2) + i) * 2 + 1] = (float)std::sin(ang);
        }
    std::vector<float> qs((size_t)Lm * d.hkv), kv((size_t)Lm * 2 * d.hkv), vs((size_t)Lm * d.hkv);
    const double log2e = 1.4426950408889634;
    for (int l = 0; l < d.L; ++l)
        for (int g = 0; g < d.hkv; ++g) {
            const float sk = fp8 ? sig[((size_t)l * 2 + 0) * d.hkv + g] : 1.0f;
            const float sv = fp8 ? sig[((size_t)l * 2 + 1) * d.hkv + g] : 1.0f;
            qs[(size_t)l * d.hkv + g] = (float)(log2e * (double)sk / std::sqrt((double)d.hd));
            kv[((size_t)l * 2 + 0) * d.hkv + g] = sk;
            kv[((size_t)l * 2 + 1) * d.hkv + g] = sv;
            vs[(size_t)l * d.hkv + g] = sv;
        }
    std::vector<double> theta((size_t)d.hd / 2);
    for (int i = 0; i < d.hd / 2; ++i) theta[i] = std::pow((double)c->plan.cfg.rope_base, -2.0 * i / d.hd);
    hipError_t e = hipMemcpyAsync(P(c, sp.rope), rope.data(), rope.size() * 4, hipMemcpyHostToDevice, st);
    if (e == hipSuccess)
        e = hipMemcpyAsync(P(c, sp.rope_theta), theta.data(), theta.size() * 8, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipMemcpyAsync(P(c, sp.qscale), qs.data(), qs.size() * 4, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipMemcpyAsync(P(c, sp.kvsig), kv.data(), kv.size() * 4, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipMemcpyAsync(P(c, sp.vscale), vs.data(), vs.size() * 4, hipMemcpyHostToDevice, st);
    // pageable sources: make sure the copies are done before the vectors die
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    return e;
}

hipEvent_t take_event(fd_ctx* c) {
    if (!c->ev_pool.empty()) {
        hipEvent_t e = c->ev_pool.back();
        c->ev_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Runs `launch` on stream st; with timing on, brackets it with events.
template <class F>
hipError_t timed(fd_ctx* c, int kind, hipStream_t st, F&& launch) {
    if (!c->prof || c->no_timing) return launch();
    hipEvent_t a = take_event(c), b = take_event(c);
    if (!a || !b) return hipErrorOutOfMemory;
    hipError_t e = hipEventRecord(a, st);
    if (e == hipSuccess) e = launch();
    if (e == hipSuccess) e = hipEventRecord(b, st);
    c->prof_pending.push_back({kind, {a, b}});
    return e;
}

// Kinds of fd_profile_read; the depth stack's projections and attention
// have kinds of their own (K_DQKV.. = K_QKV.. + kDepthKinds)
enum Kind { K_EMBED = 0, K_QKV, K_ATTN, K_O, K_GU, K_DOWN, K_FINAL, K_WIN, K_WALK, K_HEAD,
            K_DQKV, K_DATTN, K_DO, K_DGU, K_DDOWN };
constexpr int kDepthKinds = K_DQKV - K_QKV;

struct CacheRef {
    uint8_t* base;
    uint64_t slot, layer, kv, head, pos;
    int fp8;
};

// One decoder stack over the session rows already embedded in ws_x/ws_xg
// (norm partial sums in ss_a).  Leaves the residual stream in ws_x and its
// final partial sums in ss_a; returns their count through *nss_out.
hipError_t run_stack(fd_ctx* c, const fd::StackPlan& sp, const CacheRef& cache, int pos_override,
                     hipStream_t st, int* nss_out) {
    const fd::Plan& pl = c->plan;
    const fd::StackDims& d = sp.dims;
    const int wt = pl.wt;
    const bool two = wt && !pl.f16;  // projection inputs as two bf16 parts
    const float inv_d = 1.0f / (float)d.d;
    const float eps = pl.cfg.rms_eps;
    const int dk = &sp == &pl.dstack ? kDepthKinds : 0;  // profile kinds of this stack
    int nss = 1;
    hipError_t e = hipSuccess;
    for (int l = 0; l < d.L && e == hipSuccess; ++l) {
        const fd::LayerOffsets& lo = sp.layers[l];
        uint8_t* layer_cache = cache.base + (size_t)l * cache.layer;

        fd::GemmArgs g{};
        g.Sp = pl.Sp;
        g.S = pl.S;
        g.MT = pl.MT;
        g.part = (float*)Wk(c, pl.ws_part);
        g.inv_d = inv_d;
        g.eps = eps;
        g.ss_stride = pl.nss_max;
        g.f16 = pl.f16;

        // QKV projection: one plane of sums per k-split; the attention
        // kernel adds them and applies the norm, rotary and cache append
        fd::GemmArgs q = g;
        const fd::GemmShape& sq = sp.qkv;
        q.W = P(c, lo.qkv);
        q.wscale = wscale(c, lo.qkv, sp.qkv);
        q.X = Wk(c, pl.ws_xg);
        q.K = sq.K; q.KB = sq.KB; q.NB = sq.NB; q.P = sq.P; q.MG = sq.MG; q.kh = sq.kh; q.x3 = sq.x3;
        q.X_lo = two ? Wk(c, pl.ws_xg_lo) : nullptr;
        q.epi = fd::EPI_PLANES;
        q.y = (float*)Wk(c, pl.ws_qkv);
        q.ld = d.qkv_n();
        q.plane = (uint64_t)pl.Sp * d.qkv_n();
        e = timed(c, K_QKV + dk, st, [&] { return fd::launch_gemm(q, pl.wkind, sq.R, sq.MTG, sq.grid(), st); });
        if (e != hipSuccess) break;

        fd::AttnArgs at{};
        at.qkv = (const float*)Wk(c, pl.ws_qkv);
        at.P = sq.P;
        at.nqkv = d.qkv_n();
        at.plane = q.plane;
        at.ss_in = (const float*)Wk(c, pl.ws_ss_a);
        at.nss = nss;
        at.ss_stride = pl.nss_max;
        at.inv_d = inv_d;
        at.eps = eps;
        at.rope = (const float*)P(c, sp.rope);
        at.rope_theta = (const double*)P(c, sp.rope_theta);
        at.ring = pos_override < 0 && pl.ring;
        at.qscale = (const float*)P(c, sp.qscale) + (size_t)l * d.hkv;
        at.kvsig = (const float*)P(c, sp.kvsig) + (size_t)l * 2 * d.hkv;
        at.vscale = (const float*)P(c, sp.vscale) + (size_t)l * d.hkv;
        at.arena = layer_cache;
        at.slot_stride = cache.slot; at.kv_stride = cache.kv; at.head_stride = cache.head; at.pos_stride = cache.pos;
        at.active = slot_active(c);
        at.pos = slot_pos(c);
        at.order = pos_override < 0 ? slot_order(c) : nullptr;  // (depth rows: all one length)
        at.pos_override = pos_override;
        at.S = pl.S; at.hq = d.hq; at.hkv = d.hkv; at.tc = sp.attn.tc; at.n_chunks = sp.attn.n_chunks;
        at.T = d.T;
        at.MT = pl.MT;
        at.part = (float*)Wk(c, pl.ws_apart);
        at.o_out = Wk(c, pl.ws_o);
        at.o_lo = two ? Wk(c, pl.ws_o_lo) : nullptr;
        at.f16 = pl.f16;
        at.early = sp.attn.early;
        at.trace = (&sp == &pl.main && l == c->trace_layer) ? c->trace : nullptr;
        e = timed(c, K_ATTN + dk, st, [&] {
            return fd::launch_attn(at, wt, cache.fp8, d.hd, d.G(), pl.S * d.hkv * sp.attn.n_chunks, st);
        });
        if (e != hipSuccess) break;

        fd::GemmArgs o = g;
        const fd::GemmShape& so = sp.o;
        o.W = P(c, lo.o);
        o.wscale = wscale(c, lo.o, sp.o);
        o.X = Wk(c, pl.ws_o);
        o.X_lo = two ? Wk(c, pl.ws_o_lo) : nullptr;
        o.K = so.K; o.KB = so.KB; o.NB = so.NB; o.P = so.P; o.MG = so.MG; o.kh = so.kh; o.x3 = so.x3;
        o.cnt = so.fused ? (int*)Wk(c, pl.ws_cnt) : nullptr;
        o.epi = fd::EPI_RESID;
        o.x = (float*)Wk(c, pl.ws_x);
        o.xg = Wk(c, pl.ws_xg);
        o.g_next = (const float*)P(c, lo.g_ffn);
        o.xg_lo = two ? Wk(c, pl.ws_xg_lo) : nullptr;
        o.ss_out = (float*)Wk(c, pl.ws_ss_f);
        o.ld = d.d;
        e = timed(c, K_O + dk, st, [&] { return fd::launch_gemm(o, pl.wkind, so.R, so.MTG, so.grid(), st); });
        if (e != hipSuccess) break;

        fd::GemmArgs u = g;
        const fd::GemmShape& su = sp.gu;
        u.W = P(c, lo.gu);
        u.wscale = wscale(c, lo.gu, sp.gu);
        u.X = Wk(c, pl.ws_xg);
        u.K = su.K; u.KB = su.KB; u.NB = su.NB; u.P = su.P; u.MG = su.MG; u.kh = su.kh; u.x3 = su.x3;
        u.cnt = su.fused ? (int*)Wk(c, pl.ws_cnt) : nullptr;
        u.epi = fd::EPI_GU;
        u.ss_in = (const float*)Wk(c, pl.ws_ss_f);
        u.nss = so.n_groups;
        u.X_lo = two ? Wk(c, pl.ws_xg_lo) : nullptr;
        u.h_out = Wk(c, pl.ws_h);
        u.h_lo = two ? Wk(c, pl.ws_h_lo) : nullptr;
        u.F = d.f;
        e = timed(c, K_GU + dk, st, [&] { return fd::launch_gemm(u, pl.wkind, su.R, su.MTG, su.grid(), st); });
        if (e != hipSuccess) break;

        fd::GemmArgs dn = g;
        const fd::GemmShape& sd = sp.down;
        dn.W = P(c, lo.down);
        dn.wscale = wscale(c, lo.down, sp.down);
        dn.X = Wk(c, pl.ws_h);
        dn.X_lo = two ? Wk(c, pl.ws_h_lo) : nullptr;
        dn.K = sd.K; dn.KB = sd.KB; dn.NB = sd.NB; dn.P = sd.P; dn.MG = sd.MG; dn.kh = sd.kh; dn.x3 = sd.x3;
        dn.cnt = sd.fused ? (int*)Wk(c, pl.ws_cnt) : nullptr;
        dn.epi = fd::EPI_RESID;
        dn.x = (float*)Wk(c, pl.ws_x);
        dn.xg = Wk(c, pl.ws_xg);
        dn.g_next = (const float*)P(c, l + 1 < d.L ? sp.layers[l + 1].g_attn : sp.g_final);
        dn.xg_lo = two ? Wk(c, pl.ws_xg_lo) : nullptr;
        dn.ss_out = (float*)Wk(c, pl.ws_ss_a);
        dn.ld = d.d;
        e = timed(c, K_DOWN + dk, st, [&] { return fd::launch_gemm(dn, pl.wkind, sd.R, sd.MTG, sd.grid(), st); });
        nss = sd.n_groups;
    }
    *nss_out = nss;
    return e;
}

// The whole step as a persistent walk: the phase list and the argument
// blocks of every task, built once here and kept in the workspace.  Every
// phase output gets a region of its own (nothing is overwritten within a
// launch, so no XCD can hold a stale L2 line of data it reads); the caller's
// x_in, y_out and depth_out are filled in at each launch.
hipError_t build_walk(fd_ctx* c, hipStream_t s, std::string* err) {
    const fd::Plan& pl = c->plan;
    const int wt = pl.wt;
    const uint64_t Sp = pl.Sp;
    uint64_t cur = pl.ws_walk_act;
    const uint64_t end = pl.ws_walk_act + pl.walk_act_bytes;
    auto take = [&](uint64_t bytes) {
        const uint64_t o = cur;
        cur += fd::walk_region(bytes);
        return Wk(c, o);
    };
    const bool two = wt && !pl.f16;  // rows as two bf16 parts (else fp16, or fp32)
    auto take_lo = [&](uint64_t bytes) { return two ? (void*)take(bytes) : nullptr; };
    std::vector<fd::WalkPhase> phases;
    std::vector<fd::GemmArgs> gemm;
    std::vector<fd::AttnArgs> attn;
    std::vector<fd::EmbedArgs> embed;
    std::vector<fd::FinalArgs> fin;
    auto gemm_phases = [&](const fd::GemmArgs& g, const fd::GemmShape& sh) {
        const int idx = (int)gemm.size();
        gemm.push_back(g);
        phases.push_back({sh.R == 6 ? fd::WALK_GEMM6 : fd::WALK_GEMM4, idx, sh.grid(), 1});
        if (sh.P > 1 && g.epi != fd::EPI_PLANES)
            phases.push_back({sh.R == 6 ? fd::WALK_REDUCE6 : fd::WALK_REDUCE4, idx, sh.grid() / sh.P * sh.MTG, 1});
    };
    auto shaped = [&](fd::GemmArgs g, const fd::GemmShape& sh, uint64_t w_off, int d) {
        g.W = P(c, w_off);
        g.wscale = wscale(c, w_off, sh);
        g.f16 = pl.f16;
        g.K = sh.K; g.KB = sh.KB; g.NB = sh.NB; g.P = sh.P; g.MG = sh.MG;
        g.MT = pl.MT; g.Sp = pl.Sp; g.S = pl.S;
        g.ss_stride = pl.nss_max;
        g.inv_d = 1.0f / (float)d;
        g.eps = pl.cfg.rms_eps;
        g.part = sh.P > 1 && g.epi != fd::EPI_PLANES ? (float*)take(4ull * sh.part_floats) : nullptr;
        return g;
    };
    // rows entering a stack: residual x, its normed activation (bf16: two
    // parts) and the partial sums of x^2
    struct Rows {
        const float* x;
        const void* xg;
        const void* xg_lo;
        const float* ss;
        int nss;
    };
    auto embed_rows = [&](fd::EmbedArgs e, const fd::StackPlan& sp, int kind) {
        const fd::StackDims& z = sp.dims;
        e.active = slot_active(c);
        e.S = pl.S;
        e.d = z.d;
        e.MT = pl.MT;
        e.x = (float*)take(4 * Sp * z.d);
        e.xg = take(4 * Sp * z.d);
        e.xg_lo = take_lo(4 * Sp * z.d);
        e.f16 = pl.f16;
        e.g = (const float*)P(c, z.L > 0 ? sp.layers[0].g_attn : sp.g_final);
        e.ss_out = (float*)take(4 * Sp * pl.nss_max);
        e.ss_stride = pl.nss_max;
        phases.push_back({kind, (int)embed.size(), pl.Sp, 1});
        embed.push_back(e);
        return Rows{e.x, e.xg, e.xg_lo, e.ss_out, 1};
    };
    // one decoder stack's layers, as in run_stack
    auto stack = [&](const fd::StackPlan& sp, const CacheRef& cache, int pos_override, int attn_kind,
                     int combine_kind, Rows r) {
        const fd::StackDims& z = sp.dims;
        for (int l = 0; l < z.L; ++l) {
            const fd::LayerOffsets& lo = sp.layers[l];
            fd::GemmArgs q{};
            q.X = r.xg;
            q.X_lo = r.xg_lo;
            q.epi = fd::EPI_PLANES;
            q.y = (float*)take(4ull * sp.qkv.P * Sp * z.qkv_n());
            q.ld = z.qkv_n();
            q.plane = Sp * z.qkv_n();
            q = shaped(q, sp.qkv, lo.qkv, z.d);
            gemm_phases(q, sp.qkv);

            fd::AttnArgs at{};
            at.qkv = q.y;
            at.P = sp.qkv.P;
            at.nqkv = z.qkv_n();
            at.plane = q.plane;
            at.ss_in = r.ss;
            at.nss = r.nss;
            at.ss_stride = pl.nss_max;
            at.inv_d = 1.0f / (float)z.d;
            at.eps = pl.cfg.rms_eps;
            at.rope = (const float*)P(c, sp.rope);
        at.rope_theta = (const double*)P(c, sp.rope_theta);
        at.ring = pos_override < 0 && pl.ring;
            at.qscale = (const float*)P(c, sp.qscale) + (size_t)l * z.hkv;
            at.kvsig = (const float*)P(c, sp.kvsig) + (size_t)l * 2 * z.hkv;
            at.vscale = (const float*)P(c, sp.vscale) + (size_t)l * z.hkv;
            at.arena = cache.base + (size_t)l * cache.layer;
            at.slot_stride = cache.slot; at.kv_stride = cache.kv; at.head_stride = cache.head;
            at.pos_stride = cache.pos;
            at.active = slot_active(c);
            at.pos = slot_pos(c);
            at.order = pos_override < 0 ? slot_order(c) : nullptr;
            at.pos_override = pos_override;
            at.S = pl.S; at.hq = z.hq; at.hkv = z.hkv; at.tc = sp.attn.tc; at.n_chunks = sp.attn.n_chunks;
            at.T = z.T;
            at.MT = pl.MT;
            at.part = sp.attn.n_chunks > 1
                          ? (float*)take(4ull * pl.S * z.hkv * sp.attn.n_chunks * z.G() * (z.hd + 2))
                          : nullptr;
            at.o_out = take(4 * Sp * z.hq * z.hd);
            at.o_lo = take_lo(4 * Sp * z.hq * z.hd);
            at.f16 = pl.f16;
            const int ai = (int)attn.size();
            attn.push_back(at);
            phases.push_back({attn_kind, ai, pl.S * z.hkv * sp.attn.n_chunks, 1});
            if (sp.attn.n_chunks > 1) phases.push_back({combine_kind, ai, pl.S * z.hkv * z.G(), 1});

            fd::GemmArgs o{};
            o.X = at.o_out;
            o.X_lo = at.o_lo;
            o.epi = fd::EPI_RESID;
            o.x_src = r.x;
            o.x = (float*)take(4 * Sp * z.d);
            o.xg = take(4 * Sp * z.d);
            o.xg_lo = take_lo(4 * Sp * z.d);
            o.g_next = (const float*)P(c, lo.g_ffn);
            o.ss_out = (float*)take(4 * Sp * pl.nss_max);
            o.ld = z.d;
            o = shaped(o, sp.o, lo.o, z.d);
            gemm_phases(o, sp.o);

            fd::GemmArgs u{};
            u.X = o.xg;
            u.X_lo = o.xg_lo;
            u.epi = fd::EPI_GU;
            u.ss_in = o.ss_out;
            u.nss = sp.o.n_groups;
            u.h_out = take(4 * Sp * z.f);
            u.h_lo = take_lo(4 * Sp * z.f);
            u.F = z.f;
            u = shaped(u, sp.gu, lo.gu, z.d);
            gemm_phases(u, sp.gu);

            fd::GemmArgs dn{};
            dn.X = u.h_out;
            dn.X_lo = u.h_lo;
            dn.epi = fd::EPI_RESID;
            dn.x_src = o.x;
            dn.x = (float*)take(4 * Sp * z.d);
            dn.xg = take(4 * Sp * z.d);
            dn.xg_lo = take_lo(4 * Sp * z.d);
            dn.g_next = (const float*)P(c, l + 1 < z.L ? sp.layers[l + 1].g_attn : sp.g_final);
            dn.ss_out = (float*)take(4 * Sp * pl.nss_max);
            dn.ld = z.d;
            dn = shaped(dn, sp.down, lo.down, z.d);
            gemm_phases(dn, sp.down);
            r = Rows{dn.x, dn.xg, dn.xg_lo, dn.ss_out, sp.down.n_groups};
        }
        return r;
    };
    auto final_rows = [&](fd::FinalArgs f, const fd::StackPlan& sp, const Rows& r) {
        f.x = r.x;
        f.ss = r.ss;
        f.nss = r.nss;
        f.ss_stride = pl.nss_max;
        f.inv_d = 1.0f / (float)sp.dims.d;
        f.eps = pl.cfg.rms_eps;
        f.g = (const float*)P(c, sp.g_final);
        f.active = slot_active(c);
        f.S = pl.S;
        f.d = sp.dims.d;
        f.MT = pl.MT;
        return f;
    };

    // main stack
    const fd::StackPlan& mp = pl.main;
    Rows r = embed_rows(fd::EmbedArgs{}, mp, fd::WALK_EMBED_IN);
    CacheRef mc{(uint8_t*)c->buf.kv_arena, pl.kv_slot_stride, pl.kv_layer_stride, pl.kv_kv_stride,
                pl.kv_head_stride, pl.kv_pos_stride, pl.kv_fp8};
    r = stack(mp, mc, -1, fd::WALK_ATTN, fd::WALK_COMBINE, r);
    fd::FinalArgs mf = final_rows(fd::FinalArgs{}, mp, r);
    mf.ldy = mp.dims.d;
    mf.y_off = 0;
    mf.yw = pl.depth ? (void*)take(4 * Sp * mp.dims.d) : (pl.head ? (void*)Wk(c, pl.ws_yw) : nullptr);
    mf.yw_lo = two && pl.head ? (void*)Wk(c, pl.ws_yw_lo) : nullptr;
    mf.f16 = pl.f16;
    c->head_x = mf.yw;
    c->head_x_lo = mf.yw_lo;
    mf.pos = slot_pos(c);
    mf.advance = 1;
    phases.push_back({fd::WALK_FINAL_MAIN, (int)fin.size(), pl.Sp, pl.depth ? 1 : 0});
    fin.push_back(mf);

    if (pl.depth) {
        const fd::StackPlan& dp = pl.dstack;
        const fd::StackDims& dd = dp.dims;
        // input projection c = W_in y
        fd::GemmArgs g{};
        g.X = mf.yw;
        g.epi = fd::EPI_F32;
        g.y = (float*)take(4 * Sp * dd.d);
        g.ld = dd.d;
        g = shaped(g, pl.win, pl.w_in, mp.dims.d);
        gemm_phases(g, pl.win);
        const uint64_t pos_b = (uint64_t)dd.hd * 4, head_b = pos_b * dd.T, kv_b = head_b * dd.hkv,
                       layer_b = kv_b * 2, slot_b = layer_b * dd.L;
        CacheRef dc{Wk(c, pl.ws_dkv), slot_b, layer_b, kv_b, head_b, pos_b, 0};
        const float* z_prev = nullptr;
        for (int k = 0; k < dd.T; ++k) {
            fd::EmbedArgs de{};
            de.c = g.y;
            de.z = z_prev;
            Rows dr = embed_rows(de, dp, fd::WALK_EMBED);
            dr = stack(dp, dc, k, fd::WALK_ATTN_DEPTH, fd::WALK_COMBINE_DEPTH, dr);
            fd::FinalArgs f = final_rows(fd::FinalArgs{}, dp, dr);
            f.ldy = dd.T * dd.d;
            f.y_off = k * dd.d;
            f.zf = (float*)take(4 * Sp * dd.d);
            f.advance = 0;
            phases.push_back({fd::WALK_FINAL_DEPTH, (int)fin.size(), pl.Sp, k + 1 < dd.T ? 1 : 0});
            fin.push_back(f);
            z_prev = f.zf;
        }
    }
    if (cur > end || (int)phases.size() > pl.walk_max_phases || (int)gemm.size() > pl.walk_max_gemm ||
        (int)attn.size() > pl.walk_max_attn || (int)embed.size() > pl.walk_max_embed ||
        (int)fin.size() > pl.walk_max_fin) {
        *err = "walk layout exceeds its plan";
        return hipErrorInvalidValue;
    }
    // argument region: [phases][gemm][attn][embed][fin], each block 256-aligned
    std::vector<uint8_t> host(pl.walk_args_bytes, 0);
    uint64_t o = 0;
    auto put = [&](const void* src, uint64_t bytes) {
        const uint64_t at = o;
        if (bytes) std::memcpy(host.data() + at, src, bytes);
        o = fd::align_up(o + bytes);
        return at;
    };
    static_assert(sizeof(fd::GemmArgs) <= fd::kWalkArgSlot && sizeof(fd::AttnArgs) <= fd::kWalkArgSlot &&
                  sizeof(fd::EmbedArgs) <= fd::kWalkArgSlot && sizeof(fd::FinalArgs) <= fd::kWalkArgSlot,
                  "argument blocks larger than their reserved slot");
    const uint64_t ph_o = put(phases.data(), phases.size() * sizeof(fd::WalkPhase));
    const uint64_t g_o = put(gemm.data(), gemm.size() * sizeof(fd::GemmArgs));
    const uint64_t a_o = put(attn.data(), attn.size() * sizeof(fd::AttnArgs));
    const uint64_t e_o = put(embed.data(), embed.size() * sizeof(fd::EmbedArgs));
    const uint64_t f_o = put(fin.data(), fin.size() * sizeof(fd::FinalArgs));
    if (o > pl.walk_args_bytes) {
        *err = "walk arguments exceed their region";
        return hipErrorInvalidValue;
    }
    uint8_t* dev = Wk(c, pl.ws_walk_args);
    hipError_t e = hipMemcpyAsync(dev, host.data(), o, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return e;
    fd::WalkArgs& w = c->walk;
    w.phases = (const fd::WalkPhase*)(dev + ph_o);
    w.n_phases = (int)phases.size();
    w.gemm = (const fd::GemmArgs*)(dev + g_o);
    w.attn = (const fd::AttnArgs*)(dev + a_o);
    w.embed = (const fd::EmbedArgs*)(dev + e_o);
    w.fin = (const fd::FinalArgs*)(dev + f_o);
    w.x_in = nullptr;
    w.y_out = nullptr;
    w.depth_out = nullptr;
    w.bar = (unsigned*)Wk(c, pl.ws_walk_bar);
    w.abort_flag = (int*)(Wk(c, pl.ws_walk_bar) + 64);
    c->walk_shape = fd::WalkShape{wt, pl.kv_fp8 ? 1 : 0, mp.qkv.MTG, mp.dims.hd, mp.dims.G(),
                                  pl.depth ? pl.dstack.dims.hd : 0, pl.f16 ? 1 : 0};
    c->walk_grid = fd::walk_grid(c->walk_shape);
    if (c->walk_grid <= 0) {
        *err = "no co-resident grid for the walk kernel of this shape";
        return hipErrorInvalidValue;
    }
    return hipSuccess;
}

hipError_t flush_slots(fd_ctx* c, hipStream_t st) {
    if (!c->slots.dirty()) return hipSuccess;
    const int i = c->ring;
    c->ring = (c->ring + 1) % kRing;
    hipError_t e = hipSuccess;
    if (c->ev_used[i]) e = hipEventSynchronize(c->ev[i]);
    if (e != hipSuccess) return e;
    c->slots.image(c->pinned[i]);
    e = hipMemcpyAsync(c->buf.slot_table, c->pinned[i], 12ull * c->plan.S, hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return e;
    e = hipEventRecord(c->ev[i], st);
    if (e != hipSuccess) return e;
    c->ev_used[i] = true;
    c->slots.clear_dirty();
    return hipSuccess;
}

}  // namespace

extern "C" {

const char* fd_status_str(fd_status s) {
    switch (s) {
        case FD_OK: return "FD_OK";
        case FD_E_INVAL: return "FD_E_INVAL";
        case FD_E_UNSUPPORTED: return "FD_E_UNSUPPORTED";
        case FD_E_NOSLOT: return "FD_E_NOSLOT";
        case FD_E_BADSLOT: return "FD_E_BADSLOT";
        case FD_E_CTXFULL: return "FD_E_CTXFULL";
        case FD_E_DEVICE: return "FD_E_DEVICE";
        case FD_E_STATE: return "FD_E_STATE";
        default: return "FD_E_UNKNOWN";
    }
}

const char* fd_last_error(fd_ctx* ctx) { return ctx ? ctx->err.c_str() : g_global_err.c_str(); }

fd_status fd_plan(const fd_config* cfg, fd_sizes* out) {
    if (!cfg || !out) return fail(nullptr, FD_E_INVAL, "null argument");
    fd::Plan p;
    std::string err;
    fd_status st = fd::make_plan(*cfg, &p, &err);
    if (st != FD_OK) return fail(nullptr, st, err);
    out->packed_weights = p.packed_bytes;
    out->kv_arena = p.kv_bytes_total;
    out->workspace = p.workspace_bytes;
    out->slot_table = p.slot_table_bytes;
    return FD_OK;
}

fd_status fd_init(const fd_config* cfg, const fd_weights* w, const fd_buffers* buf, void* stream,
                  fd_ctx** out) {
    if (!cfg || !w || !buf || !out) return fail(nullptr, FD_E_INVAL, "null argument");
    fd::Plan p;
    std::string err;
    fd_status st = fd::make_plan(*cfg, &p, &err);
    if (st != FD_OK) return fail(nullptr, st, err);
    if (!aligned(buf->packed_weights) || !aligned(buf->kv_arena) || !aligned(buf->workspace) ||
        !aligned(buf->slot_table))
        return fail(nullptr, FD_E_INVAL, "buffers must be non-null and 256-byte aligned");
    if (p.main.dims.L > 0 && !w->layers) return fail(nullptr, FD_E_INVAL, "null layer array");
    for (int l = 0; l < p.main.dims.L; ++l)
        if (check_layer(w->layers[l]) != FD_OK) return fail(nullptr, FD_E_INVAL, "null weight pointer");
    if (!w->g_final) return fail(nullptr, FD_E_INVAL, "null g_final");
    if (p.kv_fp8 && !w->kv_scale) return fail(nullptr, FD_E_INVAL, "FP8 cache needs kv_scale");
    if (p.depth) {
        if (!w->w_in || !w->depth_g_final || (p.dstack.dims.L > 0 && !w->depth_layers))
            return fail(nullptr, FD_E_INVAL, "null depth-stack pointer");
        for (int l = 0; l < p.dstack.dims.L; ++l)
            if (check_layer(w->depth_layers[l]) != FD_OK)
                return fail(nullptr, FD_E_INVAL, "null depth weight pointer");
    }
    if (p.head && !w->w_head) return fail(nullptr, FD_E_INVAL, "vocab > 0 needs w_head");

    fd_ctx* c = new (std::nothrow) fd_ctx(p);
    if (!c) return fail(nullptr, FD_E_DEVICE, "out of host memory");
    c->buf = *buf;
    c->ws = (uint8_t*)buf->workspace;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipGetDevice(&c->device);
    for (int i = 0; i < kRing && e == hipSuccess; ++i) {
        e = hipHostMalloc((void**)&c->pinned[i], 12ull * p.S, hipHostMallocDefault);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev[i], hipEventDisableTiming);
    }
    // scales to the host (FP8 only) for the derived tables
    std::vector<float> sig;
    if (e == hipSuccess && p.kv_fp8) {
        sig.resize((size_t)p.main.dims.L * 2 * p.main.dims.hkv);
        if (!sig.empty()) {
            e = hipMemcpyAsync(sig.data(), w->kv_scale, sig.size() * 4, hipMemcpyDeviceToHost, s);
            if (e == hipSuccess) e = hipStreamSynchronize(s);
        }
        for (float v : sig)
            if (e == hipSuccess && !(v > 0.0f && std::isfinite(v))) {
                fd_destroy(c);
                return fail(nullptr, FD_E_INVAL, "kv_scale entries must be finite and > 0");
            }
    }
    if (e == hipSuccess) e = hipMemsetAsync(buf->workspace, 0, p.workspace_bytes, s);
    if (e == hipSuccess) e = hipMemsetAsync(buf->slot_table, 0, p.slot_table_bytes, s);
    if (e == hipSuccess) e = pack_stack(c, p.main, w->layers, w->g_final, s);
    if (e == hipSuccess) e = upload_tables(c, p.main, sig, p.kv_fp8, s);
    if (e == hipSuccess && p.depth) {
        e = pack(p.win, p.wt, w->w_in, p.win.N, nullptr, 0, nullptr, 0, P(c, p.w_in), s);
        if (e == hipSuccess) e = pack_stack(c, p.dstack, w->depth_layers, w->depth_g_final, s);
        if (e == hipSuccess) e = upload_tables(c, p.dstack, std::vector<float>(), false, s);
    }
    if (e == hipSuccess && p.head)
        e = pack(p.hshape, p.wkind, w->w_head, p.hshape.N, nullptr, 0, nullptr, 0, P(c, p.w_head), s);
    // the output head reads the final-normed rows (and their bf16 low part)
    c->head_x = Wk(c, p.ws_yw);
    c->head_x_lo = p.wt && !p.f16 && p.head ? Wk(c, p.ws_yw_lo) : nullptr;
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    std::string werr;
    if (e == hipSuccess && p.walk) e = build_walk(c, s, &werr);
    if (e != hipSuccess) {
        std::string msg = std::string("fd_init: ") + (werr.empty() ? hipGetErrorString(e) : werr.c_str());
        fd_destroy(c);
        return fail(nullptr, FD_E_DEVICE, msg);
    }
    c->slots.mark_dirty();
    *out = c;
    return FD_OK;
}

fd_status fd_alloc_slots(fd_ctx* c, int32_t n, int32_t* slots_out) {
    if (!c) return FD_E_INVAL;
    fd_status st = c->slots.alloc(n, slots_out);
    if (st != FD_OK) return fail(c, st, st == FD_E_NOSLOT ? "not enough free slots" : "bad argument");
    return FD_OK;
}

fd_status fd_free(fd_ctx* c, const int32_t* ids, int32_t n) {
    if (!c) return FD_E_INVAL;
    fd_status st = c->slots.free(ids, n);
    if (st != FD_OK) return fail(c, st, "invalid, unallocated or repeated slot id");
    return FD_OK;
}

fd_status fd_set_position(fd_ctx* c, int32_t slot, int32_t pos) {
    if (!c) return FD_E_INVAL;
    fd_status st = c->slots.set_position(slot, pos);
    if (st != FD_OK) return fail(c, st, "bad slot or position");
    return FD_OK;
}

fd_status fd_slot_state(fd_ctx* c, int32_t slot, int32_t* active, int32_t* pos) {
    if (!c) return FD_E_INVAL;
    fd_status st = c->slots.state(slot, active, pos);
    if (st != FD_OK) return fail(c, st, "bad slot");
    return FD_OK;
}

}  // extern "C"

namespace {

// The step of fd_step on the workspace c->ws (argument checks done by the
// callers).
fd_status step_impl(fd_ctx* c, const void* x_in, void* y_out, void* depth_out, void* stream) {
    const fd::Plan& pl = c->plan;
    int full = -1;
    if (c->slots.any_full(&full))
        return fail(c, FD_E_CTXFULL, "slot " + std::to_string(full) + " has a full window");
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = flush_slots(c, st);
    if (e != hipSuccess) return hip_fail(c, e, "slot table upload");

    if (pl.walk) {
        fd::WalkArgs w = c->walk;
        w.x_in = x_in;
        w.y_out = y_out;
        w.depth_out = depth_out;
        w.abort_init = c->walk_abort_next ? 1 : 0;
        c->walk_abort_next = false;
        e = timed(c, K_WALK, st, [&] { return fd::launch_walk(w, c->walk_shape, c->walk_grid, st); });
        if (e != hipSuccess) return hip_fail(c, e, "fd_step launch");
        c->walk_launched = true;
        c->slots.advance();
        return FD_OK;
    }

    const fd::StackPlan& mp = pl.main;
    const fd::StackDims& md = mp.dims;
    fd::EmbedArgs em{};
    em.x_in = x_in;
    em.active = slot_active(c);
    em.S = pl.S;
    em.d = md.d;
    em.MT = pl.MT;
    em.x = (float*)Wk(c, pl.ws_x);
    em.xg = Wk(c, pl.ws_xg);
    em.xg_lo = pl.wt && !pl.f16 ? Wk(c, pl.ws_xg_lo) : nullptr;
    em.f16 = pl.f16;
    em.g = (const float*)P(c, md.L > 0 ? mp.layers[0].g_attn : mp.g_final);
    em.ss_out = (float*)Wk(c, pl.ws_ss_a);
    em.ss_stride = pl.nss_max;
    e = timed(c, K_EMBED, st, [&] { return fd::launch_embed(em, pl.wt, pl.Sp, st); });
    int nss = 1;
    CacheRef mc{(uint8_t*)c->buf.kv_arena, pl.kv_slot_stride, pl.kv_layer_stride, pl.kv_kv_stride,
                pl.kv_head_stride, pl.kv_pos_stride, pl.kv_fp8};
    if (e == hipSuccess) e = run_stack(c, mp, mc, -1, st, &nss);
    if (e == hipSuccess) {
        fd::FinalArgs f{};
        f.x = (const float*)Wk(c, pl.ws_x);
        f.ss = (const float*)Wk(c, pl.ws_ss_a);
        f.nss = nss;
        f.ss_stride = pl.nss_max;
        f.inv_d = 1.0f / (float)md.d;
        f.eps = pl.cfg.rms_eps;
        f.g = (const float*)P(c, mp.g_final);
        f.active = slot_active(c);
        f.S = pl.S;
        f.d = md.d;
        f.MT = pl.MT;
        f.y_out = y_out;
        f.ldy = md.d;
        f.y_off = 0;
        f.yw = pl.depth || pl.head ? Wk(c, pl.ws_yw) : nullptr;
        f.yw_lo = pl.wt && !pl.f16 && pl.head ? Wk(c, pl.ws_yw_lo) : nullptr;
        f.f16 = pl.f16;
        f.pos = slot_pos(c);
        f.advance = 1;
        e = timed(c, K_FINAL, st, [&] { return fd::launch_final(f, pl.wt, pl.Sp, st); });
    }
    if (e == hipSuccess && pl.depth) {
        const fd::StackPlan& dp = pl.dstack;
        const fd::StackDims& dd = dp.dims;
        fd::GemmArgs g{};
        g.W = P(c, pl.w_in);
        g.X = Wk(c, pl.ws_yw);
        g.K = pl.win.K; g.KB = pl.win.KB; g.NB = pl.win.NB; g.P = pl.win.P; g.MG = pl.win.MG; g.x3 = pl.win.x3;
        g.MT = pl.MT; g.Sp = pl.Sp; g.S = pl.S;
        g.part = (float*)Wk(c, pl.ws_part);
        g.epi = fd::EPI_F32;
        g.y = (float*)Wk(c, pl.ws_c);
        g.ld = dd.d;
        e = timed(c, K_WIN, st, [&] { return fd::launch_gemm(g, pl.wt, pl.win.R, pl.win.MTG, pl.win.grid(), st); });
        const uint64_t pos_b = (uint64_t)dd.hd * 4, head_b = pos_b * dd.T, kv_b = head_b * dd.hkv,
                       layer_b = kv_b * 2, slot_b = layer_b * dd.L;
        CacheRef dc{Wk(c, pl.ws_dkv), slot_b, layer_b, kv_b, head_b, pos_b, 0};
        for (int k = 0; k < dd.T && e == hipSuccess; ++k) {
            fd::EmbedArgs de{};
            de.c = (const float*)Wk(c, pl.ws_c);
            de.z = k ? (const float*)Wk(c, pl.ws_z) : nullptr;
            de.active = slot_active(c);
            de.S = pl.S;
            de.d = dd.d;
            de.MT = pl.MT;
            de.x = (float*)Wk(c, pl.ws_x);
            de.xg = Wk(c, pl.ws_xg);
            de.g = (const float*)P(c, dd.L > 0 ? dp.layers[0].g_attn : dp.g_final);
            de.ss_out = (float*)Wk(c, pl.ws_ss_a);
            de.ss_stride = pl.nss_max;
            e = timed(c, K_EMBED, st, [&] { return fd::launch_embed(de, pl.wt, pl.Sp, st); });
            int dnss = 1;
            if (e == hipSuccess) e = run_stack(c, dp, dc, k, st, &dnss);
            if (e == hipSuccess) {
                fd::FinalArgs f{};
                f.x = (const float*)Wk(c, pl.ws_x);
                f.ss = (const float*)Wk(c, pl.ws_ss_a);
                f.nss = dnss;
                f.ss_stride = pl.nss_max;
                f.inv_d = 1.0f / (float)dd.d;
                f.eps = pl.cfg.rms_eps;
                f.g = (const float*)P(c, dp.g_final);
                f.active = slot_active(c);
                f.S = pl.S;
                f.d = dd.d;
                f.MT = pl.MT;
                f.y_out = depth_out;
                f.ldy = dd.T * dd.d;
                f.y_off = k * dd.d;
                f.zf = (float*)Wk(c, pl.ws_z);
                f.advance = 0;
                e = timed(c, K_FINAL, st, [&] { return fd::launch_final(f, pl.wt, pl.Sp, st); });
            }
        }
    }
    if (e != hipSuccess) return hip_fail(c, e, "fd_step launch");
    c->slots.advance();
    return FD_OK;
}

// Checks shared by fd_step and fd_step_static.
bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

fd_status step_args(fd_ctx* c, const void* x_in, void* y_out, void* depth_out) {
    if (!x_in || !y_out) return fail(c, FD_E_INVAL, "null x_in or y_out");
    if (c->plan.depth && !depth_out) return fail(c, FD_E_INVAL, "profile has a depth stack: depth_out required");
    // the kernels move rows in 8- and 16-byte vectors
    if (!aligned16(x_in) || !aligned16(y_out) || (depth_out && !aligned16(depth_out)))
        return fail(c, FD_E_INVAL, "x_in, y_out and depth_out must be 16-byte aligned");
    int s = -1;
    if (c->slots.any_stale(&s))
        return fail(c, FD_E_STATE, "slot " + std::to_string(s) +
                                       " is stale after a step that stopped early: fd_set_position or fd_free it");
    return FD_OK;
}

}  // namespace

namespace fd {

int ctx_device(const fd_ctx* c) { return c->device; }

// fd_step on a workspace other than the ctx's own (the library's static
// scratch): every split-counter region is cleared first, since the
// scratch holds whatever the last call on this GPU left there.
fd_status step_on_workspace(fd_ctx* c, void* ws, uint64_t ws_bytes, const void* x_in, void* y_out,
                            void* depth_out, void* stream) {
    if (!c) return FD_E_INVAL;
    fd_status st = step_args(c, x_in, y_out, depth_out);
    if (st != FD_OK) return st;
    const Plan& pl = c->plan;
    if (pl.walk)
        return fail(c, FD_E_UNSUPPORTED, "fd_step_static: FD_EXEC_WALK profiles keep their phase layout in the fd_init workspace");
    if (pl.workspace_bytes > ws_bytes)
        return fail(c, FD_E_UNSUPPORTED, "fd_step_static: the profile needs " + std::to_string(pl.workspace_bytes) +
                                             " bytes of workspace, the static scratch holds " + std::to_string(ws_bytes));
    if (!ws || ((uintptr_t)ws % kAlign)) return fail(c, FD_E_INVAL, "fd_step_static: scratch not 256-byte aligned");
    int full = -1;
    if (c->slots.any_full(&full))
        return fail(c, FD_E_CTXFULL, "slot " + std::to_string(full) + " has a full window");
    hipStream_t s = (hipStream_t)stream;
    const StackPlan* stacks[2] = {&pl.main, pl.depth ? &pl.dstack : nullptr};
    bool fused = false;
    for (const StackPlan* sp : stacks)
        if (sp) fused = fused || sp->o.fused || sp->gu.fused || sp->down.fused;
    uint8_t* saved = c->ws;
    c->ws = (uint8_t*)ws;
    c->no_timing = true;
    hipError_t e = hipSuccess;
    if (fused) {  // arrival counters of the in-kernel k-split reduction start at zero
        uint64_t cnt = 1;
        for (const StackPlan* sp : stacks)
            if (sp) for (const GemmShape* g : {&sp->o, &sp->gu, &sp->down}) cnt = std::max<uint64_t>(cnt, g->counters);
        e = launch_fill_u32((uint32_t*)Wk(c, pl.ws_cnt), 0u, cnt, s);
    }
    st = e == hipSuccess ? step_impl(c, x_in, y_out, depth_out, stream) : hip_fail(c, e, "fd_step_static");
    c->ws = saved;
    c->no_timing = false;
    return st;
}

}  // namespace fd

extern "C" {

fd_status fd_step(fd_ctx* c, const void* x_in, void* y_out, void* depth_out, void* stream) {
    if (!c) return FD_E_INVAL;
    fd_status st = step_args(c, x_in, y_out, depth_out);
    if (st != FD_OK) return st;
    return step_impl(c, x_in, y_out, depth_out, stream);
}

fd_status fd_step_tokens(fd_ctx* c, const void* x_in, void* y_out, void* depth_out, int32_t* tokens_out,
                         float* logits_out, void* stream) {
    if (!c) return FD_E_INVAL;
    const fd::Plan& pl = c->plan;
    if (!pl.head) return fail(c, FD_E_INVAL, "profile has no output head (vocab 0)");
    if (!tokens_out) return fail(c, FD_E_INVAL, "null tokens_out");
    if (((uintptr_t)tokens_out & 3) || (logits_out && !aligned16(logits_out)))
        return fail(c, FD_E_INVAL, "tokens_out must be 4-byte and logits_out 16-byte aligned");
    fd_status st = fd_step(c, x_in, y_out, depth_out, stream);
    if (st != FD_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    const fd::GemmShape& h = pl.hshape;
    fd::GemmArgs g{};
    g.W = P(c, pl.w_head);
    g.wscale = wscale(c, pl.w_head, h);
    g.X = c->head_x;
    g.X_lo = c->head_x_lo;
    g.f16 = pl.f16;
    g.K = h.K; g.KB = h.KB; g.NB = h.NB; g.P = h.P; g.MG = h.MG;
    g.MT = pl.MT; g.Sp = pl.Sp; g.S = pl.S;
    g.part = (float*)Wk(c, pl.ws_part);
    g.epi = fd::EPI_F32;
    g.y = logits_out ? logits_out : (float*)Wk(c, pl.ws_logits);
    g.ld = pl.cfg.vocab;
    fd::ArgmaxArgs am{};
    am.logits = g.y;
    am.ld = pl.cfg.vocab;
    am.V = pl.cfg.vocab;
    am.S = pl.S;
    am.active = slot_active(c);
    am.tokens = tokens_out;
    hipError_t e = timed(c, K_HEAD, s, [&] {
        hipError_t r = fd::launch_gemm(g, pl.wkind, h.R, h.MTG, h.grid(), s);
        return r == hipSuccess ? fd::launch_argmax(am, s) : r;
    });
    if (e != hipSuccess) return hip_fail(c, e, "fd_step_tokens launch");
    return FD_OK;
}

fd_status fd_kv_write(fd_ctx* c, int32_t slot, int32_t layer, int32_t t0, int32_t n, const float* src,
                      void* stream) {
    if (!c) return FD_E_INVAL;
    const fd::Plan& pl = c->plan;
    if (slot < 0 || slot >= pl.S) return fail(c, FD_E_BADSLOT, "slot out of range");
    if (layer < 0 || layer >= pl.main.dims.L) return fail(c, FD_E_INVAL, "layer out of range");
    if (n < 0 || t0 < 0 || (int64_t)t0 + n > pl.cfg.max_context)
        return fail(c, FD_E_INVAL, "positions outside the window");
    if (n == 0) return FD_OK;
    if (!src || ((uintptr_t)src & 15)) return fail(c, FD_E_INVAL, "src must be non-null and 16-byte aligned");
    fd::KvWriteArgs a{};
    a.src = src;
    a.dst = (uint8_t*)c->buf.kv_arena + (size_t)slot * pl.kv_slot_stride + (size_t)layer * pl.kv_layer_stride;
    a.kv_stride = pl.kv_kv_stride;
    a.head_stride = pl.kv_head_stride;
    a.pos_stride = pl.kv_pos_stride;
    a.kvsig = (const float*)P(c, pl.main.kvsig) + (size_t)layer * 2 * pl.main.dims.hkv;
    a.hkv = pl.main.dims.hkv;
    a.hd = pl.main.dims.hd;
    a.t0 = t0;
    a.n = n;
    a.kv_fp8 = pl.kv_fp8;
    hipError_t e = fd::launch_kv_write(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(c, e, "fd_kv_write");
    return FD_OK;
}

fd_status fd_kv_layout(fd_ctx* c, fd_kv_view* out) {
    if (!c || !out) return FD_E_INVAL;
    const fd::Plan& pl = c->plan;
    out->base = c->buf.kv_arena;
    out->slot_stride = pl.kv_slot_stride;
    out->layer_stride = pl.kv_layer_stride;
    out->kv_stride = pl.kv_kv_stride;
    out->head_stride = pl.kv_head_stride;
    out->pos_stride = pl.kv_pos_stride;
    out->elem_bytes = pl.kv_bytes;
    out->n_layers = pl.main.dims.L;
    out->n_kv_heads = pl.main.dims.hkv;
    out->max_context = pl.cfg.max_context;
    out->head_dim = pl.main.dims.hd;
    out->max_slots = pl.S;
    out->kv_scale = pl.kv_fp8 ? (const float*)P(c, pl.main.kvsig) : nullptr;
    out->slot_active = slot_active(c);
    out->slot_pos = slot_pos(c);
    return FD_OK;
}

fd_status fd_walk_abort_next(fd_ctx* c) {
    if (!c) return FD_E_INVAL;
    if (!c->plan.walk) return fail(c, FD_E_UNSUPPORTED, "fd_walk_abort_next: FD_EXEC_WALK profiles only");
    c->walk_abort_next = true;
    return FD_OK;
}

fd_status fd_trace_attention(fd_ctx* c, uint64_t* stamps, int32_t layer, int32_t max_workgroups) {
    if (!c) return FD_E_INVAL;
    if (!stamps) {
        c->trace = nullptr;
        c->trace_layer = -1;
        return FD_OK;
    }
    const fd::Plan& pl = c->plan;
    const int grid = pl.S * pl.main.dims.hkv * pl.main.attn.n_chunks;
    if (pl.walk) return fail(c, FD_E_UNSUPPORTED, "fd_trace_attention: kernel-sequence profiles only");
    if (layer < 0 || layer >= pl.main.dims.L) return fail(c, FD_E_INVAL, "layer out of range");
    if (max_workgroups < grid)
        return fail(c, FD_E_INVAL, "the stamp buffer needs " + std::to_string(grid) + " workgroups");
    if ((uintptr_t)stamps & 7) return fail(c, FD_E_INVAL, "stamps must be 8-byte aligned");
    c->trace = stamps;
    c->trace_layer = layer;
    return FD_OK;
}

fd_status fd_profile(fd_ctx* c, int32_t enable) {
    if (!c) return FD_E_INVAL;
    c->prof = enable != 0;
    return FD_OK;
}

fd_status fd_profile_read(fd_ctx* c, double* ms_out, int64_t* launches_out, int32_t n) {
    if (!c || n < 0 || (n > 0 && (!ms_out || !launches_out))) return FD_E_INVAL;
    hipError_t e = hipSuccess;
    for (auto& p : c->prof_pending) {
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventSynchronize(p.second.second);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, p.second.first, p.second.second);
        if (e == hipSuccess) {
            c->prof_ms[p.first] += ms;
            c->prof_n[p.first] += 1;
        }
        c->ev_pool.push_back(p.second.first);
        c->ev_pool.push_back(p.second.second);
    }
    c->prof_pending.clear();
    for (int k = 0; k < n && k < FD_N_KINDS; ++k) {
        ms_out[k] = c->prof_ms[k];
        launches_out[k] = c->prof_n[k];
    }
    for (int k = 0; k < FD_N_KINDS; ++k) {
        c->prof_ms[k] = 0.0;
        c->prof_n[k] = 0;
    }
    if (e != hipSuccess) return hip_fail(c, e, "fd_profile_read");
    return FD_OK;
}

fd_status fd_sync(fd_ctx* c, void* stream) {
    if (!c) return FD_E_INVAL;
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(c, e, "fd_sync");
    if (c->walk_launched) {
        int flag = 0;
        e = hipMemcpy(&flag, c->walk.abort_flag, sizeof(int), hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_fail(c, e, "fd_sync");
        c->walk_launched = false;
        if (flag) {
            c->slots.mark_stale();
            return fail(c, FD_E_DEVICE, "walk: a grid barrier wait timed out; the active slots are stale");
        }
    }
    return FD_OK;
}

fd_status fd_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, int32_t grid, void* stream) {
    if (!buf || !sink || grid < 1 || bytes < 16 || ((uintptr_t)buf & 15)) return FD_E_INVAL;
    hipError_t e = fd::launch_read_probe(buf, bytes, sink, grid, (hipStream_t)stream);
    return e == hipSuccess ? FD_OK : FD_E_DEVICE;
}

fd_status fd_destroy(fd_ctx* c) {
    if (!c) return FD_E_INVAL;
    for (auto& p : c->prof_pending) {
        (void)hipEventSynchronize(p.second.second);
        (void)hipEventDestroy(p.second.first);
        (void)hipEventDestroy(p.second.second);
    }
    for (hipEvent_t e : c->ev_pool) (void)hipEventDestroy(e);
    for (int i = 0; i < kRing; ++i) {
        if (c->ev[i]) {
            if (c->ev_used[i]) (void)hipEventSynchronize(c->ev[i]);
            (void)hipEventDestroy(c->ev[i]);
        }
        if (c->pinned[i]) (void)hipHostFree(c->pinned[i]);
    }
    delete c;
    return FD_OK;
}

}  // extern "C"
