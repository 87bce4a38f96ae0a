// Kernel argument blocks and launchers of the decode step (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fd {

enum Epilogue : int {
    EPI_PLANES = 0, // split ks stores its unnormalised sums to plane ks of y (the attention kernel
                    // adds the planes, applies the norm, rotary and cache append)
    EPI_RESID = 1,  // x += acc; xg = act(x * g_next); per-row partial sums of x^2
    EPI_GU = 2,     // rows x rstd, h = silu(gate) * up
    EPI_F32 = 3,    // plain fp32 store
};

struct GemmArgs {
    const uint8_t* W;   // packed tiles [NB][KB][64 lanes][16 B]
    const void* X;      // session rows [Sp][K], activation type, fragment-packed layout
    const void* X_lo;   // optional (bf16 only): low parts, the input being X + X_lo
    int K, KB, NB, P, MG, MT, Sp, S;
    float* part;        // split-K partial tiles (P > 1): [n-group*MG + m-group][P][tiles][64][4]
    int* cnt;           // P > 1, non-null: per (n-group, m-group) arrival counters (zero between
                        // launches); the last workgroup to arrive adds the partials and finishes
    int epi;
    // row scaling by the RMS norm of the GEMM input: rstd[m] = (sum_i ss[i][m] / d + eps)^-1/2
    const float* ss_in;    // [Sp][ss_stride] partial sums of x^2 of the GEMM input rows
    int nss, ss_stride;
    float inv_d, eps;
    // EPI_PLANES
    uint64_t plane;        // floats between consecutive split planes of y
    // EPI_RESID
    float* x;              // [Sp][ld] residual stream (written)
    const float* x_src;    // residual input when not x itself (persistent walk), else null
    void* xg;              // [Sp][ld] act(x * g_next)
    void* xg_lo;           // optional (bf16): x * g_next - xg, rounded to bf16
    const float* g_next;
    float* ss_out;         // [Sp][ss_stride], entry n-group
    int ld;
    // EPI_GU
    void* h_out;           // [Sp][F]
    void* h_lo;            // optional (bf16): h - h_out, rounded to bf16
    int F;
    // EPI_F32 / EPI_PLANES
    float* y;              // [Sp][ld] (EPI_PLANES: [P][Sp][ld])
    const float* wscale;   // FP8 or fp16 weight codes: [NB*16] output-row scales (the tiles hold
                           // codes of w / scale)
    int kh;                // row-split variant: k-halves per workgroup (1 or 2; 0 = 1)
    int f16;               // 2-byte stacks: X is one fp16 part (weights FP8 or fp16 codes), and
                           // the epilogue stores xg / h as fp16; else bf16
    int x3;                // fp32 stacks: W holds bf16 high and low parts of the fp32 weights
                           // (tiles of 16 rows x 32 k, see pack3_kernel) and the products are
                           // three bf16 ones per k-step (lo*hi + hi*lo + hi*hi of weight*row)
};

struct AttnArgs {
    // QKV projection of this layer: P split planes [P][Sp][nqkv] of
    // unnormalised sums, columns [q heads | k heads | v heads] x hd
    const float* qkv;
    int P, nqkv;
    uint64_t plane;
    // attention-norm row scale: rstd[s] = (sum_i ss[s][i] / d + eps)^-1/2
    const float* ss_in;
    int nss, ss_stride;
    float inv_d, eps;
    const float* rope;     // [T][hd/2] x (cos, sin)
    const float* qscale;   // [hkv] log2(e) * sigma_K / sqrt(hd) of this layer
    const float* kvsig;    // [2][hkv] FP8 scales of this layer (1 for fp32 caches)
    const float* vscale;   // [hkv] sigma_V of this layer
    uint8_t* arena;        // cache base of this layer for slot 0
    uint64_t slot_stride, kv_stride, head_stride, pos_stride;
    const int* active;
    const int* pos;
    const int* order;      // or null: task row r runs slot order[r] (a permutation of the
                           // slots, longest windows first); null: slot r
    int pos_override;      // >= 0: every row is at this position (depth stack)
    int S, hq, hkv, tc, n_chunks;
    int T;                 // cache positions per slot
    int ring;              // rolling window: frame p at cache position p % T, the last T frames attended
    const double* rope_theta;  // [hd/2] base^(-2i/hd): rotary angles of frames p >= T (rolling window)
    int MT;                // 16-row tiles of session rows (packed output layout)
    float* part;           // [S][hkv][n_chunks][G][hd + 2]
    void* o_out;           // [Sp][hq*hd] activation type, fragment-packed
    void* o_lo;            // optional (bf16): o - o_out, rounded to bf16
    int f16;               // 2-byte stacks: o_out is fp16 (one part)
    int early;             // request each wave's first block of keys/values before the prologue
    uint64_t* trace;       // optional: 4 device-clock stamps per workgroup [grid][4]
                           // (entry, prologue done, stream done, exit)
};

struct EmbedArgs {
    const void* x_in;      // caller rows [S][d] (activation type), or null
    const float* c;        // depth input projection [Sp][d] fp32 (when x_in is null)
    const float* z;        // previous depth output [Sp][d] fp32 or null (= 0)
    const int* active;
    int S, d, MT;
    float* x;              // [Sp][d]
    void* xg;              // [Sp][d]
    void* xg_lo;           // optional (bf16): x * g - xg, rounded to bf16
    int f16;               // 2-byte stacks: xg is fp16 (one part)
    const float* g;        // gain of the first norm
    float* ss_out;         // [Sp][ss_stride], entry 0
    int ss_stride;
};

struct FinalArgs {
    const float* x;
    const float* ss;       // [Sp][ss_stride]
    int nss, ss_stride;
    float inv_d, eps;
    const float* g;
    const int* active;
    int S, d, MT;
    void* y_out;           // caller rows, element (m, i) at y_out[m * ldy + y_off + i]; may be null
    int ldy, y_off;
    void* yw;              // [Sp][d] activation-type copy (GEMM input layout), or null
    void* yw_lo;           // optional (bf16): y - yw, rounded to bf16 (output head input)
    int f16;               // 2-byte stacks: yw is fp16 (one part)
    float* zf;             // [Sp][d] fp32 copy, or null
    int* pos;              // advanced by one for active rows when `advance`
    int advance;
};

// Greedy token per row: argmax over logits[m][0..V) (ties to the lowest
// index), -1 for inactive rows.
struct ArgmaxArgs {
    const float* logits;   // [S..][ld]
    int ld, V, S;
    const int* active;
    int32_t* tokens;       // [S]
};

struct PackArgs {
    const void* src[3];
    int rows[3];
    int interleave;        // 1: packed row 2j = src0 row j, 2j+1 = src1 row j
    int N, K, KB;
    uint8_t* dst;
    float* scale;          // FP8 / fp16 weight codes: per packed row, max|w| / 448 or a power of
                           // two (see row_scale_kernel; 1 for a zero row)
    int f16;               // 1: fp16 codes (power-of-two scales)
    int x3;                // fp32 source split into bf16 high and low tiles (KB: k-tiles of 32)
};

struct KvWriteArgs {
    const float* src;      // [2][hkv][n][hd]
    uint8_t* dst;          // slot + layer base
    uint64_t kv_stride, head_stride, pos_stride;
    const float* kvsig;    // [2][hkv]
    int hkv, hd, t0, n, kv_fp8;
};

// Persistent walk: one cooperative launch runs a list of phases, each over
// n_items workgroup tasks (the bodies of the separate kernels), with a grid
// barrier after every phase whose outputs a later one reads.
enum WalkKind : int {
    WALK_GEMM4 = 0, WALK_GEMM6, WALK_REDUCE4, WALK_REDUCE6,
    WALK_ATTN, WALK_COMBINE,               // main stack attention (and chunk merge)
    WALK_ATTN_DEPTH, WALK_COMBINE_DEPTH,   // depth stack attention
    WALK_EMBED,                            // rows from EmbedArgs (depth input c + z)
    WALK_EMBED_IN,                         // rows of the launch's x_in
    WALK_FINAL_MAIN,                       // final norm into the launch's y_out, positions advance
    WALK_FINAL_DEPTH                       // final norm of a depth step into the launch's depth_out
};

struct WalkPhase {
    int kind, idx, n_items, barrier;
};

struct WalkArgs {
    const WalkPhase* phases;
    int n_phases;
    const GemmArgs* gemm;
    const AttnArgs* attn;
    const EmbedArgs* embed;
    const FinalArgs* fin;
    const void* x_in;      // the caller's buffers of this step
    void* y_out;
    void* depth_out;
    unsigned* bar;         // barrier counter, zeroed before the launch
    int* abort_flag;       // set when a barrier wait times out
    int abort_init;        // value the flag starts at (1: every workgroup leaves at its first
                           // barrier wait, the abort path forced from the host)
};

// Shape a walk kernel is compiled for: weight / cache types, m-tiles per
// GEMM m-group, head_dim and query heads per kv head of the main stack,
// head_dim of the depth stack (0: none), and (2-byte stacks) whether the
// projections take their rows as one fp16 part (else two bf16 parts).
struct WalkShape {
    int wt, fp8, MTG, hd, G, dhd, f16;
};

// Depth of a GEMM wave's register ring of k-tiles: as deep as ~48
// outstanding 16-byte-per-lane loads allow (the wave's load counter holds
// 63), at least 2.  SX: the session rows come as two bf16 parts.
constexpr int gemm_stages(int NG, int MTG, int SX = 0, int W8 = 0) {
    return 48 / (NG + (1 + W8) * MTG * (1 + SX)) < 2
               ? 2
               : (48 / (NG + (1 + W8) * MTG * (1 + SX)) > 8 ? 8 : 48 / (NG + (1 + W8) * MTG * (1 + SX)));
}
// Ring depth of the three-product fp32 loop: a stage holds 2 * (NG + MTG)
// 16-byte fragments; as many stages as ~232 registers allow next to the
// accumulators and the split rows, at least 2, at most 8.
constexpr int x3_stages(int NG, int MTG) {
    return (232 - 4 * NG * MTG - 8) / (8 * (NG + MTG)) < 2
               ? 2
               : ((232 - 4 * NG * MTG - 8) / (8 * (NG + MTG)) > 8 ? 8 : (232 - 4 * NG * MTG - 8) / (8 * (NG + MTG)));
}

// Launchers (enqueue on `st`; return the launch error).
hipError_t launch_pack(const PackArgs& a, int wt, hipStream_t st);
hipError_t launch_gemm(const GemmArgs& a, int wt, int NG, int MTG, int grid, hipStream_t st);
hipError_t launch_attn(const AttnArgs& a, int wt, int kv_fp8, int hd, int G, int grid, hipStream_t st);
hipError_t launch_embed(const EmbedArgs& a, int wt, int rows, hipStream_t st);
hipError_t launch_final(const FinalArgs& a, int wt, int rows, hipStream_t st);
hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t st);
hipError_t launch_argmax(const ArgmaxArgs& a, hipStream_t st);
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, int grid, hipStream_t st);
// Sets n 32-bit words at p to v (a kernel, so it can sit inside a captured graph).
hipError_t launch_fill_u32(uint32_t* p, uint32_t v, uint64_t n, hipStream_t st);
// Persistent walk: walk_grid() is the co-resident grid of the shape's
// compiled kernel (0 if the shape has none); launch_walk() zeroes the
// barrier state and launches.
int walk_grid(const WalkShape& s);
hipError_t launch_walk(const WalkArgs& w, const WalkShape& s, int grid, hipStream_t st);

}  // namespace fd
