// Serving-profile validation and layout planning (pure host code).
#include "fd_plan.h"

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <sstream>

namespace fd {

GemmShape shape_with(int N, int K, int KT, int MT, int NG, int P, int cap = kMaxMTG) {
    GemmShape g;
    g.N = N;
    g.K = K;
    g.KT = KT;
    g.NB = N / 16;
    g.KB = K / KT;
    g.MG = cdiv(MT, cap);
    g.MTG = cdiv(MT, g.MG);
    g.R = NG;
    g.P = P;
    g.n_groups = cdiv(g.NB, NG);
    g.part_floats = P > 1 ? (uint64_t)g.n_groups * g.MG * P * NG * g.MTG * 256 : 0;
    g.counters = g.n_groups * g.MG;
    return g;
}

// A split must divide the k-tiles evenly and leave each of a workgroup's
// four waves at least one.
bool valid_split(const GemmShape& g, int P) {
    return P >= 1 && g.KB % P == 0 && g.KB / P >= 4;
}

GemmShape choose_gemm(int N, int K, int KT, int MT, int n_cu, int cap, bool small, bool x3) {
    // Candidates: 6 or 4 weight blocks per workgroup (6 only while the
    // accumulators of a 5-tile m-group fit; small: also 2, which fills as
    // many CUs with half the splits), any split P that gives every wave at
    // least one step.  Score: how evenly the grid fills whole rounds of one
    // workgroup per CU, minus a small charge per extra split (its partial
    // tiles cost a write and a read); ties keep more blocks per workgroup.
    GemmShape best = shape_with(N, K, KT, MT, 4, 1, cap);
    double best_score = -1e9;
    for (int NG : {6, 4, 2}) {
        GemmShape base = shape_with(N, K, KT, MT, NG, 1, cap);
        if (NG == 6 && (base.MTG > 5 || x3)) continue;
        if (NG == 2 && !(small && small_blocks_ok(2, base.MTG))) continue;
        for (int P = 1; P <= 64; ++P) {
            if (!valid_split(base, P)) continue;
            GemmShape g = shape_with(N, K, KT, MT, NG, P, cap);
            const int grid = g.grid();
            const int rounds = cdiv(grid, n_cu);
            const double fill = (double)grid / ((double)rounds * n_cu);
            double score = fill - 0.04 * (P - 1) - (rounds > 2 ? 0.1 : 0.0);
            if (grid < n_cu / 2) score -= 0.3;
            if (score > best_score + 1e-9) {
                best_score = score;
                best = g;
            }
        }
    }
    // Two or one weight blocks per workgroup with no or 2 k-splits (small:
    // fp32 stacks in the kernel sequence).  Each activation k-tile is then
    // fetched once per 2 or 1 blocks rather than once per 4-6, which pays
    // where it removes most of the split (no reduce launch, fewer planes
    // for attention to add) and still fills two thirds of the CUs in at
    // most two rounds: the first of (2 blocks, no split), (1, no split),
    // (1, 2 splits) that does; with the three-product loop, whose products
    // cost less per block, (2 blocks, 2 splits) comes second.
    if (small && best.P > 1) {
        const int cand_f32[3][2] = {{2, 1}, {1, 1}, {1, 2}};
        const int cand_x3[4][2] = {{2, 1}, {2, 2}, {1, 1}, {1, 2}};
        const int (*cand)[2] = x3 ? cand_x3 : cand_f32;
        const int n_cand = x3 ? 4 : 3;
        for (int i = 0; i < n_cand; ++i) {
            const int* c = cand[i];
            if (c[0] == best.R && c[1] == best.P) break;  // the score's choice comes first
            if (c[1] >= best.P) continue;
            GemmShape g = shape_with(N, K, KT, MT, c[0], c[1], cap);
            if (small_blocks_ok(c[0], g.MTG) && valid_split(g, c[1]) && 3 * g.grid() >= 2 * n_cu &&
                g.grid() <= 2 * n_cu)
                return g;
        }
    }
    return best;
}

namespace {

bool valid_hd(int hd) { return hd == 64 || hd == 128 || hd == 256; }

fd_status check_stack(const char* name, int L, int d, int hq, int hkv, int hd, int f, int KT,
                      std::string* err) {
    std::ostringstream m;
    if (L < 0 || L > 1024) m << name << ": n_layers " << L << " outside 0..1024";
    else if (d <= 0 || d % (8 * KT)) m << name << ": d_model " << d << " must be a positive multiple of " << 8 * KT;
    else if (d > 65536) m << name << ": d_model too large";
    else if (hq <= 0 || hkv <= 0 || hq % hkv) m << name << ": n_heads must be a positive multiple of n_kv_heads";
    else if (!(hq / hkv == 1 || hq / hkv == 2 || hq / hkv == 4))
        m << name << ": n_heads / n_kv_heads must be 1, 2 or 4";
    else if (!valid_hd(hd)) m << name << ": head_dim must be 64, 128 or 256";
    else if ((hq * hd) % (8 * KT)) m << name << ": n_heads*head_dim must be a multiple of " << 8 * KT;
    else if (f <= 0 || f % (8 * KT) || f > 262144)
        m << name << ": d_ffn must be a positive multiple of " << 8 * KT;
    if (!m.str().empty()) {
        *err = m.str();
        return FD_E_UNSUPPORTED;
    }
    return FD_OK;
}

// Tuning override for measurements: FD_TUNE="qkv.P=4,o.NG=4,attn.chunks=2"
// replaces the chosen split-K factor (P) or n-blocks per workgroup (NG) of
// a projection ("d.gu.P=1": of the depth stack's), or the attention chunk
// count; "fused=1" (or "o.fused=1")
// makes the last workgroup of each n-group add the k-split partials
// instead of a reduce launch (measured slower at 80 sessions: 9.76 vs
// 9.43 ms per step).  Unset in normal use.
int tune_value(const char* key, int dflt) {
    const char* env = std::getenv("FD_TUNE");
    if (!env) return dflt;
    std::string s(env), k = std::string(key) + "=";
    size_t p = 0;
    while ((p = s.find(k, p)) != std::string::npos) {
        if (p == 0 || s[p - 1] == ',') return std::atoi(s.c_str() + p + k.size());
        p += k.size();
    }
    return dflt;
}

GemmShape tuned(GemmShape g, const char* name, bool ns, int cap, bool small, bool x3) {
    std::string n(name);
    int NG = tune_value((n + ".NG").c_str(), g.R);
    int P = tune_value((n + ".P").c_str(), g.P);
    if (!(NG == 4 || (NG == 6 && g.MTG <= 5 && !x3) || (ns && ns_blocks_ok(NG, g.MTG)) ||
          (small && small_blocks_ok(NG, g.MTG))))
        NG = g.R;
    GemmShape base = shape_with(g.N, g.K, g.KT, g.MG * g.MTG, NG, 1, cap);
    if (!valid_split(base, P)) P = valid_split(base, g.P) ? g.P : 1;
    GemmShape out = shape_with(g.N, g.K, g.KT, g.MG * g.MTG, NG, P, cap);
    if (ns_blocks_ok(NG, out.MTG)) {
        const int kh = tune_value((n + ".KH").c_str(), g.kh);
        out.kh = kh == 2 && (out.KB / P) % 2 == 0 ? 2 : 1;
    }
    out.fused = P > 1 && NG <= 6 && tune_value((n + ".fused").c_str(), tune_value("fused", 0)) != 0;
    out.x3 = x3 ? 1 : 0;
    return out;
}

// pre: prefix of the stack's tuning keys ("" main, "d." depth stack)
// scaled: the packed matrices carry per-row scales (FP8 or fp16 codes)
// small: the 1- and 2-block fp32 kernels may be chosen (kernel sequence);
// x3: the fp32 projections run the three-product loop on tiles of 32 k
void plan_stack(StackPlan& sp, const StackDims& dims, int KT, int MT, int S, int kv_fp8, bool w8,
                bool scaled, uint64_t& off, bool ns, bool small, bool x3, const std::string& pre) {
    sp.dims = dims;
    const int cap = (w8 || x3) ? kMaxMTG8 : kMaxMTG;
    const int kt = x3 ? 32 : KT;
    auto pick = [&](int N, int K, const char* name) {
        return tuned(choose_gemm(N, K, kt, MT, 256, cap, small, x3), (pre + name).c_str(), ns, cap, small, x3);
    };
    sp.qkv = pick(dims.qkv_n(), dims.d, "qkv");
    sp.o = pick(dims.d, dims.hq * dims.hd, "o");
    sp.gu = pick(2 * dims.f, dims.d, "gu");
    sp.down = pick(dims.d, dims.f, "down");
    sp.layers.resize(dims.L);
    auto tiles = [scaled](const GemmShape& g) { return packed_matrix_bytes(g, scaled); };
    for (int l = 0; l < dims.L; ++l) {
        LayerOffsets& lo = sp.layers[l];
        lo.qkv = off; off = align_up(off + tiles(sp.qkv));
        lo.o = off;   off = align_up(off + tiles(sp.o));
        lo.gu = off;  off = align_up(off + tiles(sp.gu));
        lo.down = off; off = align_up(off + tiles(sp.down));
        lo.g_attn = off; off = align_up(off + 4ull * dims.d);
        lo.g_ffn = off;  off = align_up(off + 4ull * dims.d);
    }
    sp.g_final = off; off = align_up(off + 4ull * dims.d);
    int Lm = std::max(dims.L, 1);
    sp.qscale = off; off = align_up(off + 4ull * Lm * dims.hkv);
    sp.kvsig = off;   off = align_up(off + 4ull * Lm * 2 * dims.hkv);
    sp.vscale = off; off = align_up(off + 4ull * Lm * dims.hkv);
    sp.rope = off;   off = align_up(off + 4ull * dims.T * dims.hd);
    sp.rope_theta = off; off = align_up(off + 8ull * dims.hd / 2);
    // attention chunking: lanes per position give each lane 16 bytes (FP8)
    // or 32 bytes (fp32) of a position's head vector
    // Chunks of the window per (slot, kv head): one workgroup per chunk.
    // A single chunk (no merge kernel) when the slot x head pairs alone give
    // about four workgroups per CU; otherwise enough chunks to get there,
    // but no chunk shorter than ~512 KiB of keys and values (per-workgroup
    // set-up and merge costs would dominate).  Chunks are whole wave loads
    // of positions.
    AttnShape& a = sp.attn;
    a.lpp = kv_fp8 ? dims.hd / 16 : dims.hd / 8;
    const int round = kWaves * (kv_fp8 ? kAttnItersFp8 : kAttnIters) * (64 / a.lpp);
    const int pairs = std::max(1, S * dims.hkv);
    const int64_t window_bytes = (int64_t)dims.T * 2 * dims.hd * (kv_fp8 ? 1 : 4);
    int want = std::max(1, std::min(cdiv(1024, pairs), (int)((window_bytes + (512 << 10) - 1) >> 19)));
    // Fewer pairs than resident workgroups (two per CU): enough chunks of at
    // least 256 KiB to fill them in one round (the talker's 56 sessions x 1
    // kv head: 9 chunks, 504 workgroups, 6.39 against 6.48 ms per step with 7)
    want = std::max(want, std::min(512 / pairs, (int)(window_bytes >> 18)));
    want = std::max(1, tune_value("attn.chunks", want));
    const int ppl = 64 / a.lpp;  // positions per wave load
    a.tc = want == 1 ? cdiv(dims.T, round) * round : cdiv(cdiv(dims.T, want), ppl) * ppl;
    // the merge kernel holds one chunk per thread: at most 256 chunks
    a.tc = std::max(a.tc, cdiv(cdiv(dims.T, 256), round) * round);
    a.n_chunks = cdiv(dims.T, a.tc);
    a.early = tune_value("attn.early", 0);
}

}  // namespace

fd_status make_plan(const fd_config& c, Plan* out, std::string* err) {
    Plan p;
    p.cfg = c;
    if (!(c.w_dtype == FD_F32 || c.w_dtype == FD_BF16 || c.w_dtype == FD_FP8_E4M3)) {
        *err = "w_dtype must be FD_F32, FD_BF16 or FD_FP8_E4M3";
        return FD_E_UNSUPPORTED;
    }
    if (c.act_dtype != (c.w_dtype == FD_FP8_E4M3 ? FD_BF16 : c.w_dtype)) {
        *err = "act_dtype must equal w_dtype (FD_BF16 with FD_FP8_E4M3 weights)";
        return FD_E_UNSUPPORTED;
    }
    if (c.w_dtype == FD_FP8_E4M3 && (c.depth_steps > 0 || c.exec_mode == FD_EXEC_WALK)) {
        *err = "FD_FP8_E4M3 weights: no depth stack and no FD_EXEC_WALK";
        return FD_E_UNSUPPORTED;
    }
    if (!(c.kv_dtype == FD_F32 || c.kv_dtype == FD_FP8_E4M3)) {
        *err = "kv_dtype must be FD_F32 or FD_FP8_E4M3";
        return FD_E_UNSUPPORTED;
    }
    if (c.vocab < 0 || c.vocab > (1 << 20) || c.vocab % 16) {
        *err = "vocab must be 0 (no output head) or a multiple of 16 up to 2^20";
        return FD_E_UNSUPPORTED;
    }
    if (!(c.proj_in == FD_PROJ_AUTO || c.proj_in == FD_PROJ_F16 || c.proj_in == FD_PROJ_BF16X2)) {
        *err = "proj_in must be FD_PROJ_AUTO, FD_PROJ_F16 or FD_PROJ_BF16X2";
        return FD_E_UNSUPPORTED;
    }
    if (c.proj_in != FD_PROJ_AUTO && c.act_dtype != FD_BF16) {
        *err = "proj_in applies to FD_BF16 profiles (fp32 profiles take FD_PROJ_AUTO)";
        return FD_E_UNSUPPORTED;
    }
    if (c.kv_ring != 0 && c.kv_ring != 1) {
        *err = "kv_ring must be 0 (fixed window) or 1 (rolling window)";
        return FD_E_INVAL;
    }
    if (c.exec_mode != FD_EXEC_KERNELS && c.exec_mode != FD_EXEC_WALK) {
        *err = "exec_mode must be FD_EXEC_KERNELS or FD_EXEC_WALK";
        return FD_E_INVAL;
    }
    if (!(c.rms_eps >= 0.0f) || !std::isfinite(c.rms_eps)) {
        *err = "rms_eps must be finite and >= 0";
        return FD_E_INVAL;
    }
    if (!(c.rope_base > 0.0f) || !std::isfinite(c.rope_base)) {
        *err = "rope_base must be finite and > 0";
        return FD_E_INVAL;
    }
    if (c.max_slots < 1 || c.max_slots > 4096) {
        *err = "max_slots outside 1..4096";
        return FD_E_UNSUPPORTED;
    }
    if (c.max_context < 1 || c.max_context > 65536) {
        *err = "max_context outside 1..65536";
        return FD_E_UNSUPPORTED;
    }
    p.wt = c.act_dtype == FD_BF16 ? 1 : 0;
    p.w8 = c.w_dtype == FD_FP8_E4M3;
    p.f16 = p.wt && c.proj_in != FD_PROJ_BF16X2;
    p.wkind = p.w8 ? 2 : (p.f16 ? 3 : p.wt);
    p.act_bytes = p.wt ? 2 : 4;
    p.kv_fp8 = c.kv_dtype == FD_FP8_E4M3;
    p.ring = c.kv_ring == 1;
    p.head = c.vocab > 0;
    p.kv_bytes = p.kv_fp8 ? 1 : 4;
    const int KT = p.w8 ? 64 : (p.wt ? 32 : 16);  // k per weight tile
    fd_status st = check_stack("main", c.n_layers, c.d_model, c.n_heads, c.n_kv_heads, c.head_dim,
                               c.d_ffn, KT, err);
    if (st != FD_OK) return st;
    p.depth = c.depth_steps > 0;
    if (c.depth_steps < 0 || c.depth_steps > 64) {
        *err = "depth_steps outside 0..64";
        return FD_E_UNSUPPORTED;
    }
    if (p.depth) {
        if (p.wt || p.kv_fp8) {
            *err = "the depth stack requires fp32 weights and an fp32 cache";
            return FD_E_UNSUPPORTED;
        }
        st = check_stack("depth", c.depth_layers, c.depth_d, c.depth_heads, c.depth_kv_heads,
                         c.depth_head_dim, c.depth_ffn, KT, err);
        if (st != FD_OK) return st;
    }
    p.S = c.max_slots;
    // fp32 stacks in the kernel sequence: one- and two-block projections;
    // the three-product loop only on request (FD_TUNE "x3=1": ~16-bit
    // operands, not the exact fp32 products the fp32 path is defined by)
    const bool small = c.exec_mode == FD_EXEC_KERNELS && !p.wt;
    const bool x3 = small && tune_value("x3", 0) != 0;
    // session rows padded to whole m-groups (at most kMaxMTG 16-row tiles
    // each, kMaxMTG8 with FP8 weights or the three-product loop) so the GEMM
    // main loop needs no row checks
    p.MT = padded_mtiles(c.max_slots, (p.w8 || x3) ? kMaxMTG8 : kMaxMTG);
    p.Sp = p.MT * 16;

    uint64_t off = 0;
    StackDims md{c.n_layers, c.d_model, c.n_heads, c.n_kv_heads, c.head_dim, c.d_ffn, c.max_context};
    // the row-split projection variant: bf16 weights (two-part or fp16
    // rows), launched as kernels (the persistent walk runs gemm_wg)
    const bool ns = c.exec_mode == FD_EXEC_KERNELS && p.wt && !p.w8;
    const bool scaled = p.wkind >= 2;
    plan_stack(p.main, md, KT, p.MT, p.S, p.kv_fp8, p.w8, scaled, off, ns, small, x3, "");
    if (p.depth) {
        StackDims dd{c.depth_layers, c.depth_d, c.depth_heads, c.depth_kv_heads, c.depth_head_dim,
                     c.depth_ffn, c.depth_steps};
        p.win = x3 ? choose_gemm(c.depth_d, c.d_model, 32, p.MT, 256, kMaxMTG8, small, true)
                   : choose_gemm(c.depth_d, c.d_model, KT, p.MT, 256);
        p.win.x3 = x3 ? 1 : 0;
        p.w_in = off;
        off = align_up(off + packed_matrix_bytes(p.win, false));
        plan_stack(p.dstack, dd, KT, p.MT, p.S, 0, false, false, off, false, small, x3, "d.");
    }
    if (p.head) {
        p.hshape = choose_gemm(c.vocab, c.d_model, KT, p.MT, 256, p.w8 ? kMaxMTG8 : kMaxMTG);
        p.w_head = off;
        off = align_up(off + packed_matrix_bytes(p.hshape, scaled));
    }
    p.packed_bytes = std::max<uint64_t>(off, kAlign);

    // workspace
    const StackDims& m = p.main.dims;
    int dmax = m.d, hqd = m.hq * m.hd, fmax = m.f, dd = 0;
    if (p.depth) {
        const StackDims& z = p.dstack.dims;
        dmax = std::max(dmax, z.d);
        hqd = std::max(hqd, z.hq * z.hd);
        fmax = std::max(fmax, z.f);
        dd = z.d;
    }
    uint64_t Sp = p.Sp;
    uint64_t w = 0;
    auto take = [&](uint64_t bytes) { uint64_t o = w; w = align_up(w + std::max<uint64_t>(bytes, 4)); return o; };
    p.ws_x = take(Sp * dmax * 4);
    p.ws_xg = take(Sp * dmax * p.act_bytes);
    // QKV projection planes, one per k-split: [P][Sp][(hq + 2 hkv) hd] fp32
    uint64_t qkv_floats = (uint64_t)p.main.qkv.P * Sp * p.main.dims.qkv_n();
    if (p.depth)
        qkv_floats = std::max(qkv_floats, (uint64_t)p.dstack.qkv.P * Sp * p.dstack.dims.qkv_n());
    p.ws_qkv = take(qkv_floats * 4);
    p.ws_o = take(Sp * hqd * p.act_bytes);
    p.ws_h = take(Sp * fmax * p.act_bytes);
    // bf16 low parts of every projection input (FD_PROJ_BF16X2): each GEMM
    // takes its session rows as two bf16 parts (hi + lo, ~16 significant
    // bits), so the activations between phases lose little more than fp32
    // rounding would
    const bool two = p.wt && !p.f16;
    p.ws_xg_lo = take(two ? Sp * dmax * 2 : 0);
    p.ws_h_lo = take(two ? Sp * fmax * 2 : 0);
    p.ws_o_lo = take(two ? Sp * hqd * 2 : 0);
    p.ws_yw = take(Sp * m.d * p.act_bytes);
    p.ws_yw_lo = take(two && p.head ? Sp * m.d * 2 : 0);
    p.ws_logits = take(p.head ? Sp * (uint64_t)c.vocab * 4 : 0);
    p.ws_c = take(Sp * std::max(dd, 1) * 4);
    p.ws_z = take(Sp * std::max(dd, 1) * 4);
    int nss = 1;
    uint64_t part = 0;
    int cnt = 1;
    uint64_t apart = 0;
    int acnt = 1;
    auto acc_stack = [&](const StackPlan& s) {
        nss = std::max({nss, s.o.n_groups, s.down.n_groups});
        for (const GemmShape* g : {&s.o, &s.gu, &s.down}) {  // (QKV splits write planes)
            part = std::max(part, g->part_floats);
            cnt = std::max(cnt, g->counters);
        }
        apart = std::max(apart, (uint64_t)p.S * s.dims.hkv * s.attn.n_chunks * s.dims.G() *
                                    (s.dims.hd + 2));
        acnt = std::max(acnt, p.S * s.dims.hkv);
    };
    acc_stack(p.main);
    if (p.depth) {
        acc_stack(p.dstack);
        part = std::max(part, p.win.part_floats);
        cnt = std::max(cnt, p.win.counters);
    }
    if (p.head) {
        part = std::max(part, p.hshape.part_floats);
        cnt = std::max(cnt, p.hshape.counters);
    }
    p.nss_max = nss;
    p.ws_ss_a = take(4ull * nss * Sp);
    p.ws_ss_f = take(4ull * nss * Sp);
    p.ws_part = take(4ull * part);
    p.ws_cnt = take(4ull * cnt);
    p.ws_apart = take(4ull * apart);
    p.ws_acnt = take(4ull * acnt);
    if (p.depth) {
        const StackDims& z = p.dstack.dims;
        p.ws_dkv = take(Sp * z.L * 2ull * z.hkv * z.T * z.hd * 4);
        p.dstack.kv_off = p.ws_dkv;
    }
    p.walk = c.exec_mode == FD_EXEC_WALK;
    if (p.walk) {
        const StackDims& m = p.main.dims;
        const int dhd = p.depth ? p.dstack.dims.hd : 0, dG = p.depth ? p.dstack.dims.G() : 0;
        if (!walk_shape_compiled(p.wt, p.kv_fp8, p.main.qkv.MTG, m.hd, m.G(), dhd, dG) ||
            (p.depth && p.dstack.qkv.MTG != p.main.qkv.MTG)) {
            *err = "FD_EXEC_WALK is compiled for: fp32 with head_dim 64, G 1, no depth stack, <= 32 "
                   "slots; fp32 with head_dim 256, G 4 and a depth stack of head_dim 128, G 1, <= 64 "
                   "slots; bf16 weights with an FP8 cache, head_dim 128, G 1, no depth stack, <= 5 row "
                   "tiles per m-group (<= 80 slots, or > 128)";
            return FD_E_UNSUPPORTED;
        }
        // every cross-phase output gets a region of its own; sizes at 4 bytes
        // per element (2-byte rows use half); two-part rows add low parts
        const uint64_t f4 = 4;
        const int lo = p.wt && !p.f16 ? 1 : 0;
        auto stack_layer = [&](const StackPlan& sp) {
            const StackDims& z = sp.dims;
            uint64_t b = 0;
            b += walk_region(f4 * sp.qkv.P * Sp * z.qkv_n());                      // QKV planes
            b += (1 + lo) * walk_region(f4 * Sp * z.hq * z.hd);                  // o (+ low part)
            if (sp.attn.n_chunks > 1)
                b += walk_region(f4 * p.S * z.hkv * sp.attn.n_chunks * z.G() * (z.hd + 2));
            for (const GemmShape* g : {&sp.o, &sp.gu, &sp.down})
                if (g->P > 1) b += walk_region(f4 * g->part_floats);                // k-split partials
            // x, xg (+ low part), ss after O and after down
            b += 2 * ((2 + lo) * walk_region(f4 * Sp * z.d) + walk_region(f4 * Sp * p.nss_max));
            b += (1 + lo) * walk_region(f4 * Sp * z.f);                           // h (+ low part)
            return b;
        };
        auto stack_in = [&](const StackDims& z) {   // embed: x, xg (+ low part), ss
            return (2 + lo) * walk_region(f4 * Sp * z.d) + walk_region(f4 * Sp * p.nss_max);
        };
        p.walk_act_bytes = stack_in(m) + (uint64_t)m.L * stack_layer(p.main);
        p.walk_max_gemm = 4 * m.L;
        p.walk_max_attn = m.L;
        p.walk_max_embed = 1;
        p.walk_max_fin = 1;
        p.walk_max_phases = 2 + m.L * 9;
        if (p.depth) {
            const StackDims& z = p.dstack.dims;
            p.walk_act_bytes += walk_region(f4 * Sp * m.d) + walk_region(f4 * Sp * z.d);  // y (W_in input), c
            if (p.win.P > 1) p.walk_act_bytes += walk_region(f4 * p.win.part_floats);
            p.walk_act_bytes += (uint64_t)z.T * (stack_in(z) + walk_region(f4 * Sp * z.d) +  // z_k
                                                 (uint64_t)z.L * stack_layer(p.dstack));
            p.walk_max_gemm += 1 + z.T * z.L * 4;
            p.walk_max_attn += z.T * z.L;
            p.walk_max_embed += z.T;
            p.walk_max_fin += z.T;
            p.walk_max_phases += 2 + z.T * (2 + z.L * 9);
        }
        const int slots = p.walk_max_gemm + p.walk_max_attn + p.walk_max_embed + p.walk_max_fin;
        p.walk_args_bytes = align_up((uint64_t)slots * kWalkArgSlot + (uint64_t)p.walk_max_phases * 16);
        p.ws_walk_act = take(p.walk_act_bytes);
        p.ws_walk_args = take(p.walk_args_bytes);
        p.ws_walk_bar = take(256);
    }
    p.ws_err = take(64);
    p.workspace_bytes = w;

    // cache arena: [S][L][K|V][H_kv][T][D]
    p.kv_pos_stride = (uint64_t)m.hd * p.kv_bytes;
    p.kv_head_stride = p.kv_pos_stride * m.T;
    p.kv_kv_stride = p.kv_head_stride * m.hkv;
    p.kv_layer_stride = p.kv_kv_stride * 2;
    p.kv_slot_stride = p.kv_layer_stride * m.L;
    p.kv_bytes_total = std::max<uint64_t>(p.kv_slot_stride * p.S, kAlign);
    p.slot_table_bytes = align_up(12ull * p.S);  // active, pos, attention task order
    *out = p;
    return FD_OK;
}

}  // namespace fd
