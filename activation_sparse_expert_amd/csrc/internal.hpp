// Host-side declarations shared by the C ABI (api.cpp) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moeffn {

// Everything the sparse expert kernel needs, passed by value.
struct SparseArgs {
    uint32_t dec_mask, dec_one;         // INT2 decode constants (set by the launcher)
    int d, f;
    int cpw;                            // channels per workgroup tile
    int tiles;                          // workgroups per token chunk
    int slots;                          // token-chunk slots in the grid
    const uint8_t *up_q;                // expert 0 of a fixed-stride pool
    const uint16_t *up_sz;
    const uint16_t *gate;
    const uint16_t *down;
    size_t q_stride, sz_stride, w_stride;   // per-expert strides (elements)
    const float *thr_dev;               // [E+S] or nullptr
    float thr;                          // single-expert threshold
    const uint16_t *x;                  // [T][d]
    int T;
    // single-expert mode
    const float *token_scale;           // [T] or nullptr
    // layer mode (layer != 0)
    int layer, E, k, S;
    const int32_t *chunk_tab;           // routed chunks: expert << 16 | first grouped position
    const int32_t *chunk_rec;           // single-token chunks: [chunk] {expert, pair, weight bits, position}
    const int32_t *n_chunks;            // [1] routed chunks in chunk_tab
    const int32_t *offset;              // [E+1]
    const int32_t *pairs;               // [T*k]
    const float *topk_w;                // [T*k]
    // single-token layer calls with route != 0: each routed workgroup ranks
    // the token's logits itself (no grouping step).  route_lg: the E logits,
    // bias included, from the logits kernel; nullptr: the workgroup forms
    // them from route_w [E][d] (type rdt) and route_bias.
    int route;
    const float *route_lg;
    const void *route_w;
    int rdt;
    const float *route_bias;
    int renorm;
    // trace exports of such calls, written by the workgroup of slot 0, tile 0
    int32_t *ex_topk_idx;               // [k]
    float *ex_topk_w;                   // [k]
    float *ex_logits;                   // [E]
    int32_t *ex_count;                  // [E]
    int32_t *ex_eam_row;                // [E], incremented
    // outputs
    float *part;                        // partial rows [rows][part_stride][d] (workspace)
    int part_stride;                    // partial slots per row (0: tiles)
    uint8_t *mask_out;                  // single: [T][f]; layer: [T][k+S][f]
    float *v_out;                       // single only: [T][f]
};


// Launch the fused Algorithm-1 kernel; tb = tokens per chunk (1, 2, 4).
hipError_t launch_sparse_expert_f16(const SparseArgs &a, int tb, hipStream_t s);
hipError_t launch_sparse_expert_bf16(const SparseArgs &a, int tb, hipStream_t s);
// the same kernel with the up codes at bits = 8, 4 or 1 (plain packing, d = 512 ... 4096)
hipError_t launch_sparse_expert_bits(const SparseArgs &a, int bits, bool bf16, int tb, hipStream_t s);

// Second kernel: output rows from the partial rows.
constexpr int kMaxExpertsPerToken = 1024;   // k + S of a layer (routed + shared rows per token)

struct ReduceArgs {
    const float *part;                  // [rows][stride][d]; a row's first slots hold its partials
    int tiles, d, T;
    int stride;                         // partial slots per row (0: tiles)
    int layer;                          // 0: row of token t is t; 1: routed + shared rows
    int rows_per_tok;                   // 1 or k + S
    int k, S;
    void *y;
    int ydt;
    int accumulate;
    // path chosen per expert (mix != 0, layer): a routed row holds tiles_dense
    // partials when its expert took the dense path (expert_dense[topk_idx]),
    // else tiles; the shared rows hold tiles_dense when shared_dense
    int mix, tiles_dense, shared_dense;
    const int32_t *topk_idx;
    const uint8_t *expert_dense;
};
hipError_t launch_reduce(const ReduceArgs &a, hipStream_t s);

struct RouteArgs {
    const void *x;
    int xdt;
    int T, d;
    const void *rw;
    int rdt;
    const float *bias;
    int E, k, renorm;
    int32_t *topk_idx;
    float *topk_w;
    float *logits;                      // nullable
    int32_t *count, *offset, *pairs;    // nullable as a group (grouping skipped)
    int32_t *active, *n_active;         // nullable
    int chunk;                          // > 0: split each expert's pairs into chunks of this size
    int32_t *chunk_tab, *n_chunks;      // [<= T*k], [1]: expert << 16 | first grouped position
    float *lg_buf;                      // [T][E] workspace for the wide-router split (route_split)
    int32_t *chunk_rec;                 // nullable, with chunk == 1: [T*k][4] per-chunk records
    int32_t *eam_row;                   // nullable: [E] per-expert counts are added into it
    // path chosen per expert (dense_min > 0): experts with at least dense_min
    // pairs go to the dense kernels, listed in chunks of dense_chunk
    int dense_min, dense_chunk;
    int32_t *chunk_tab2, *n_chunks2;    // dense chunks
    uint8_t *expert_dense;              // nullable: [E] 1 where the expert took the dense path
};
// Routers with more than 8 experts whose rows are large per token (E d
// element bytes above 32 KB) compute their logits in a separate kernel spread
// over many workgroups.
bool route_split(int d, int E, int rdt);
hipError_t launch_route(const RouteArgs &a, hipStream_t s);
// the logits alone (a.lg_buf [T][E], bias included), for inline routing
hipError_t launch_route_logits(const RouteArgs &a, hipStream_t s);
// single-token layer calls route inside the expert kernel; routers up to this
// size are read there by every routed workgroup, larger ones by the logits kernel
constexpr size_t kInlineRouterBytes = 64u << 10;

struct DenseArgs {
    int d, f, E, k, S, T;
    const uint16_t *x;                  // [T][d] bf16
    const uint16_t *gate, *up, *down;   // [E+S][f][d] bf16
    const int32_t *active, *n_active, *offset, *pairs;
    const float *topk_w;
    float *h;                           // [T*(k+S)][f] fp32 intermediate (workspace)
    float *part;                        // [T*(k+S)][kDenseKSplit][d] partial rows (workspace)
};
constexpr int kDenseKSplit = 4;         // split of the intermediate dimension in the down GEMM
hipError_t launch_dense_layer(const DenseArgs &a, hipStream_t s);
size_t dense_h_bytes(int T, int f, int k, int S);

hipError_t launch_pack_int2(const void *w, int dt, int d, int f, uint8_t *q, uint16_t *sz,
                            hipStream_t s);
hipError_t launch_materialize16(const uint8_t *q, const uint16_t *sz, int d, int f, bool bf16,
                                uint16_t *out, hipStream_t s);

// Dense grouped GEMM (dense_gemm.hip): gate/up then down for a layer, token
// rows in chunks of at most 256 of one expert (the grouping kernel's chunk
// table), W^down transposed ([d][f]) for the down product.
struct GemmArgs {
    int d, f, E, k, S, T;
    int bf16;                           // 1: bf16 MFMA, 0: fp16
    const uint16_t *x;                  // [T][d]
    const uint16_t *gate, *up;          // [E+S][f][d]
    const uint16_t *down_t;             // [E+S][d][f]
    uint16_t *h16;                      // [T (k + S)][f] workspace, 16-bit
    float *part;                        // [T (k + S)][part_stride][d] partial rows
    int part_stride;                    // partial slots per row (0: ksplit)
    const int32_t *chunk_tab, *n_chunks, *offset, *pairs;
    const float *topk_w;
    int ksplit;                         // split of f in the down product
    int grid_chunks;                    // chunk slots in the grid (an upper bound)
    int mt;                             // token rows per chunk and tile: 256 or 64
};
constexpr int kGemmChunk = 256;         // token rows per chunk (64 or 128 for experts with fewer tokens)
int gemm_grid_chunks(int T, int k, int E, int S, int mt);
hipError_t launch_gemm_layer(const GemmArgs &a, hipStream_t s);
// out [mats][cols][rows] = in [mats][rows][cols], 16-bit elements
hipError_t launch_transpose16(const uint16_t *in, int mats, int rows, int cols, uint16_t *out,
                              hipStream_t s);
hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s);
hipError_t launch_fill_u8(uint8_t *p, size_t n, uint8_t v, hipStream_t s);
// Bitmask and population count of `rows` 0/1 byte masks of f channels (f % 64
// == 0): bits [rows][f/64] (channel 64 i + l at bit l of word i) and nnz [rows];
// either may be null.
hipError_t launch_mask_bits(const uint8_t *m, int rows, int f, uint64_t *bits, int32_t *nnz,
                            hipStream_t s);

// Up codes at 8, 4 or 1 bits (plain packing) and the group-64 scales.
hipError_t launch_pack_bits(const void *w, int dt, int d, int f, int bits, uint8_t *q,
                            uint16_t *sz, hipStream_t s);

// Cosine-distance nearest stored EAM: dist [n] fp64 (written), idx_out [1].
hipError_t launch_eamc_match(const int32_t *eamc, int n, int len, const int32_t *query,
                             int32_t *idx_out, double *dist, hipStream_t s);

// Threshold calibration: out = linear-interpolation quantile of |v| between
// order statistics r_lo and r_hi with weight gamma (computed on the host).
size_t calibrate_ws_bytes();
hipError_t launch_calibrate(const float *v, long long n, long long r_lo, long long r_hi,
                            double gamma, float *out, void *ws, hipStream_t s);

}  // namespace moeffn
