// Host-side plan of one serving profile: tiling of every projection,
// attention chunking, and the byte layout of the packed-weight buffer and
// the workspace.  Pure host code (no HIP): compiled into the HIP library
// and into the host-only test library.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/fd.h"

namespace fd {

constexpr int kWaves = 4;          // waves per workgroup in the GEMM and attention kernels
constexpr int kTileBytes = 1024;   // one packed weight tile = 64 lanes x 16 bytes
constexpr int kMaxMTG = 8;         // most 16-row tiles of sessions one GEMM workgroup holds
constexpr int kMaxMTG8 = 5;        // (FP8 weights: the kernels are built for up to 5)
constexpr int kAttnIters = 4;      // position loads per attention wave block (fp32 cache)
constexpr int kAttnItersFp8 = 8;   // (FP8 cache)
constexpr uint64_t kAlign = 256;

inline uint64_t align_up(uint64_t v, uint64_t a = kAlign) { return (v + a - 1) / a * a; }
inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// Tiling of one projection Y[M][N] = X[M][K] . W[N][K]^T.
struct GemmShape {
    int N = 0, K = 0;
    int KT = 0;        // k-width of a tile: 32 (bf16) or 16 (fp32)
    int NB = 0, KB = 0;  // tiles along N (16 rows each) and K
    int R = 4;         // n-blocks per workgroup: 4 or 6 shared by its 4 k-split waves, or
                       // 8, 12 or 16 split between its waves (row-split variant, bf16)
    int P = 1;         // k-splits (workgroups sharing one n-group)
    int MG = 1;        // m-groups
    int MTG = 1;       // 16-row m-tiles per m-group
    int n_groups = 0;  // ceil(NB / R)
    uint64_t w_off = 0;   // offset of the packed tiles in the packed buffer
    uint64_t part_floats = 0;  // partial-sum floats needed when P > 1 (n_groups*MG*P*R*MTG*256)
    int counters = 0;
    bool fused = false;  // P > 1: the last workgroup of an n-group adds the partials (no reduce launch)
    int kh = 1;          // row-split variant: k-halves per workgroup (2: two waves per SIMD)
    int x3 = 0;          // fp32 weights as bf16 high and low tiles of 32 k (2 KiB per tile),
                         // three bf16 products per k-step (kernel sequence)
    int grid() const { return n_groups * P * MG; }
};

struct StackDims {
    int L = 0, d = 0, hq = 0, hkv = 0, hd = 0, f = 0;
    int T = 0;          // cache positions per slot (window / depth steps)
    int G() const { return hkv ? hq / hkv : 0; }
    int qkv_n() const { return (hq + 2 * hkv) * hd; }
};

struct LayerOffsets {
    uint64_t qkv = 0, o = 0, gu = 0, down = 0;  // packed tiles
    uint64_t g_attn = 0, g_ffn = 0;              // fp32 gains
};

struct AttnShape {
    int lpp = 0;      // lanes per position
    int tc = 0;       // positions per chunk (one workgroup)
    int n_chunks = 0; // chunks per (slot, kv-head) for a full window
    int early = 0;    // first block of the stream requested before the prologue
    uint64_t part_floats = 0;
};

struct StackPlan {
    StackDims dims;
    GemmShape qkv, o, gu, down;
    AttnShape attn;
    std::vector<LayerOffsets> layers;
    uint64_t g_final = 0;  // fp32 [d]
    uint64_t qscale = 0;   // fp32 [L][H_kv]: log2(e) * sigma_K / sqrt(D)
    uint64_t kvsig = 0;    // fp32 [L][2][H_kv]: FP8 scale sigma (1 for fp32 caches)
    uint64_t vscale = 0;   // fp32 [L][H_kv]: sigma_V
    uint64_t rope = 0;     // fp32 [T][D/2][2] (cos, sin)
    uint64_t rope_theta = 0;  // float64 [D/2] base^(-2i/D): angles past the table (rolling window)
    // workspace (per stack) cache for the depth stack
    uint64_t kv_off = 0;
};

struct Plan {
    fd_config cfg{};
    bool ring = false;  // rolling window (kv_ring = 1)
    bool head = false;  // output head (vocab > 0)
    GemmShape hshape;   // output head projection
    uint64_t w_head = 0;  // packed offset of the head tiles
    int wt = 0;       // 1 = bf16 activations (bf16 or FP8 weights), 0 = fp32
    bool w8 = false;  // FP8 E4M3 weights with per-output-row scales
    bool f16 = false; // 2-byte stack with fp16 projection inputs (FD_PROJ_F16), else two bf16
                      // parts (FD_PROJ_BF16X2)
    int wkind = 0;    // weight format of the projections: 0 fp32, 1 bf16, 2 FP8 codes, 3 fp16 codes
                      // (2 and 3 with per-row scales after the tiles)
    int act_bytes = 4;
    int kv_fp8 = 0;
    int kv_bytes = 4;
    int S = 0;        // max_slots
    int Sp = 0;       // S rounded up to 16
    int MT = 0;       // Sp / 16
    bool depth = false;
    StackPlan main, dstack;
    GemmShape win;    // depth input projection
    uint64_t w_in = 0;

    // packed-weight buffer
    uint64_t packed_bytes = 0;
    // workspace layout
    uint64_t ws_x = 0, ws_xg = 0, ws_qkv = 0, ws_o = 0, ws_h = 0, ws_c = 0, ws_z = 0, ws_yw = 0;
    uint64_t ws_ss_a = 0, ws_ss_f = 0, ws_part = 0, ws_cnt = 0, ws_apart = 0, ws_acnt = 0;
    uint64_t ws_dkv = 0, ws_err = 0, ws_xg_lo = 0, ws_h_lo = 0, ws_o_lo = 0;
    uint64_t ws_yw_lo = 0, ws_logits = 0;  // head input low part (bf16), logits [Sp][vocab]
    // persistent walk (the whole step as one launch): whether it is used,
    // and its workspace regions
    bool walk = false;
    uint64_t ws_walk_act = 0, ws_walk_args = 0, ws_walk_bar = 0;
    uint64_t walk_act_bytes = 0, walk_args_bytes = 0;
    int walk_max_gemm = 0, walk_max_attn = 0, walk_max_embed = 0, walk_max_fin = 0,
        walk_max_phases = 0;
    int nss_max = 0;
    uint64_t workspace_bytes = 0;
    // cache arena
    uint64_t kv_slot_stride = 0, kv_layer_stride = 0, kv_kv_stride = 0, kv_head_stride = 0,
             kv_pos_stride = 0;
    uint64_t kv_bytes_total = 0;
    uint64_t slot_table_bytes = 0;
};

// Validates cfg and builds the plan.  Returns FD_OK or an error code with
// a message in *err.
fd_status make_plan(const fd_config& cfg, Plan* out, std::string* err);

// Bytes of one walk buffer region: every cross-phase output of the walk has
// a region of its own (no L2 line of it can be stale in another XCD).
inline uint64_t walk_region(uint64_t bytes) { return align_up(bytes > 0 ? bytes : 4); }

// Shapes the persistent walk kernel is compiled for: fp32 stacks with
// head_dim 64, one query head per kv head and no depth stack (up to 2
// m-tiles); fp32 stacks with head_dim 256, 4 query heads per kv head and a
// depth stack of head_dim 128 with one query head per kv head (up to 4);
// bf16 weights with an FP8 cache, head_dim 128, one query head per kv head,
// no depth stack (up to 5).
inline bool walk_shape_compiled(bool wt, bool fp8, int MTG, int hd, int G, int dhd, int dG) {
    if (!wt && !fp8 && hd == 64 && G == 1 && dhd == 0) return MTG >= 1 && MTG <= 2;
    if (!wt && !fp8 && hd == 256 && G == 4 && dhd == 128 && dG == 1) return MTG >= 1 && MTG <= 4;
    if (wt && fp8 && hd == 128 && G == 1 && dhd == 0) return MTG >= 1 && MTG <= 5;
    return false;
}

// Bytes per argument block reserved in the walk's argument region.
constexpr uint64_t kWalkArgSlot = 512;

// Bytes of one projection's packed weights: the tiles, then (FP8 or fp16
// codes) one fp32 scale per output row.
inline uint64_t packed_matrix_bytes(const GemmShape& g, bool scaled) {
    return (uint64_t)g.NB * g.KB * kTileBytes * (g.x3 ? 2 : 1) + (scaled ? 4ull * g.NB * 16 : 0);
}

// Tile choice for one projection (exposed for tests).
// cap: most m-tiles per m-group (kMaxMTG, or kMaxMTG8 for FP8 weights).
// small: one or two weight blocks per workgroup may be chosen (fp32 kernel
// sequence); x3: the three-product fp32 loop (no 6-block shapes).
GemmShape choose_gemm(int N, int K, int KT, int MT, int n_cu, int cap = kMaxMTG, bool small = false,
                      bool x3 = false);

// Session rows padded to whole m-groups of at most `cap` 16-row tiles.
inline int padded_mtiles(int slots, int cap) {
    const int mt = cdiv(slots, 16);
    const int mg = cdiv(mt, cap);
    return mg * cdiv(mt, mg);
}

// Row-split projection variant (bf16 weights, two-part activations): 8, 12
// or 16 blocks per workgroup (2, 3 or 4 per wave), at most 5 m-tiles.
inline bool ns_blocks_ok(int NG, int MTG) { return (NG == 8 || NG == 12 || NG == 16) && MTG <= 5; }
// One or two weight blocks per workgroup (fp32 weights, kernel sequence):
// built for m-groups of up to 5 tiles.
inline bool small_blocks_ok(int NG, int MTG) { return (NG == 1 || NG == 2) && MTG <= 5; }

}  // namespace fd
