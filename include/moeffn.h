/*
 * libmoeffn — activation-sparse MoE expert FFN for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every buffer argument is a plain device pointer (memory from
 * hipMalloc or a PyTorch CUDA/HIP tensor) unless a comment says "host".
 * Descriptor structs (moe_expert_view, moe_layer, moe_layer_trace) are host
 * structs whose pointer fields are device pointers.
 *
 * What is computed (sources are reviews of the papers, cited by page title and
 * section):
 *   FloE review, "MoE 专家前向计算": a SwiGLU expert computes
 *       a_E(x) = (SiLU(x W^gate) (.) x W^up) W^down.
 *   FloE review, "混合压缩策略": gate and down are activation-sparsified, up
 *       is stored in INT2.
 *   FloE review, "高效稀疏 GEMV 内核" (Algorithm 1 and the optimisations after
 *       it): v = x W^up, mask = |v| > t, x' = SiLU(x W^gate[mask]) (.) v[mask],
 *       output = x' W^down_T with W^down transposed so that only the selected
 *       rows are read, SiLU fused with the product.
 *   MoE-Infinity review, "A3 背景" and MoE-Lightning review, "MoE 模型架构":
 *       a router sends each token to its top-k experts.
 *   MoE-Infinity review, "4.3": per layer, the number of tokens routed to each
 *       expert (one row of the expert activation matrix).
 *
 * Data layout (all row-major, one expert):
 *   up_q   [f][d/4]   uint8: INT2 codes of W^up, row j = output channel j.
 *                     A row is d/16 little-endian 32-bit words; word i holds
 *                     inputs 16i..16i+15, the code of input 16i + 2m + h
 *                     (m = 0..7, h = 0/1) in bits 16h + 2m (even inputs in the
 *                     low half-word, odd inputs in the high half-word).
 *   up_sz  [f][d/64][2] fp16 bits {s, z}: for group g = k/64 of channel j the
 *                     up weight is w = s * (q - z).
 *   gate_t [f][d]     row j = column j of W^gate (fp16 or bf16).
 *   down   [f][d]     row j = row j of W^down, i.e. W^down transposed and stored
 *                     column-major, so an active channel's row is contiguous.
 * A layer stores its E routed experts then its S shared experts back to back at
 * a fixed per-expert stride in each of these four arrays.
 *
 * Constraints checked on the host before anything is enqueued:
 *   d a multiple of 64 from 64 to 16384;
 *   f % 64 == 0;  T >= 1;
 *   activations and gate/down weights have the same 16-bit type (fp16 or bf16);
 *   16-byte aligned up_q/gate_t/down/x and 4-byte aligned up_sz.
 *
 * Workspace: every forward call takes a device workspace of at least
 * moe_workspace_size(...) bytes (fp32 partial rows, routing tables and, for
 * routers with more than 8 experts, the [T][E] fp32 router logits).  It
 * needs no initialisation and holds nothing from one call to the next.  Calls
 * that share a workspace must be ordered (same stream); overlapping calls need
 * distinct workspaces.
 *
 * Execution: calls are asynchronous on `stream` (a hipStream_t passed as void*,
 * NULL = the null stream).  Forward calls do no host synchronisation and no
 * device-to-host copy.  The library allocates nothing and keeps no pointer
 * after a call returns.
 *
 * Errors: invalid arguments return a negative moe_status and enqueue nothing;
 * a failed kernel launch returns MOE_ERR_HIP.  No C++ exception crosses the ABI.
 *
 * Determinism: routing, grouping, masks, v and y are bit-reproducible for the
 * same inputs and shapes.  Each workgroup writes its share of y as an fp32
 * partial row and a second kernel sums the partial rows in a fixed order; no
 * floating-point atomics are used.
 */
#ifndef MOEFFN_H
#define MOEFFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums are int-sized in C and C++ alike.  C++ callers (and the library
 * itself) see them with a fixed int underlying type, so that any int a caller
 * passes is a valid value of the type and is rejected by the argument checks
 * rather than being undefined. */
#ifdef __cplusplus
#define MOE_ENUM enum : int
#else
#define MOE_ENUM enum
#endif

typedef MOE_ENUM {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,   /* null pointer, bad size, k outside [1, E], ... */
    MOE_ERR_UNSUPPORTED = -2,   /* shape or dtype combination not implemented    */
    MOE_ERR_ALIGNMENT = -3,     /* a pointer is not aligned as required          */
    MOE_ERR_WORKSPACE = -4,     /* workspace missing or smaller than required    */
    MOE_ERR_HIP = -5            /* a HIP runtime call or kernel launch failed    */
} moe_status;

typedef MOE_ENUM { MOE_F16 = 0, MOE_BF16 = 1, MOE_F32 = 2 } moe_dtype;

typedef MOE_ENUM {
    MOE_PATH_SPARSE = 0,        /* Algorithm 1: INT2 up, threshold mask, row gathers */
    MOE_PATH_DENSE = 1,         /* MFMA grouped GEMM (bf16, fp16), threshold off    */
    MOE_PATH_AUTO = 2,          /* per call: the path with the lower expected time  */
    MOE_PATH_MIXED = 3          /* per expert: dense from a token count, in one call */
} moe_path;

typedef MOE_ENUM {
    MOE_OP_EXPERT = 0,          /* moe_expert_forward_sparse */
    MOE_OP_ROUTE = 1,           /* moe_route_topk           */
    MOE_OP_LAYER = 2,           /* moe_layer_forward        */
    MOE_OP_CALIBRATE = 3,       /* moe_calibrate_threshold  */
    MOE_OP_EAMC = 4,            /* moe_eamc_match (T = n, d = len) */
    MOE_OP_EXPERT_BITS = 5      /* moe_expert_forward_sparse_bits, any width */
} moe_op;

/* One compressed expert (FloE review, "混合压缩策略": {W^S(gate), W^S(down),
 * W^Q(up)}; Algorithm 1 inputs E_ij and t_ij). */
typedef struct {
    const uint8_t *up_q;        /* [f][d/4]        */
    const uint16_t *up_sz;      /* [f][d/64][2]    */
    const void *gate_t;         /* [f][d] wdt      */
    const void *down;           /* [f][d] wdt      */
    float threshold;            /* channel j is active iff |v_j| > threshold (fp32);
                                   t < 0 keeps all channels, +inf keeps none */
} moe_expert_view;

/* One MoE layer: E routed experts (top-k) followed by S shared experts (always
 * applied with weight 1), all in the compressed format at a fixed stride. */
typedef struct {
    int d, f;                   /* hidden size, intermediate size          */
    int n_routed, n_shared;     /* E, S (k + S <= 1024)                     */
    int top_k;                  /* k, 1 <= k <= E                           */
    int renormalize;            /* 1: softmax over the k chosen logits;
                                   0: full softmax taken at the chosen ones */
    moe_dtype wdt;              /* gate/down (and activation) type          */
    const void *router_w;       /* [E][d] in rdt                            */
    moe_dtype rdt;
    const float *router_bias;   /* [E] or NULL                              */
    const uint8_t *up_q;        /* [E+S][f][d/4]                            */
    const uint16_t *up_sz;      /* [E+S][f][d/64][2]                        */
    const void *gate_t;         /* [E+S][f][d]                              */
    const void *down;           /* [E+S][f][d]                              */
    const float *thresholds;    /* [E+S] fp32, device                       */
    const uint16_t *up_dense;   /* [E+S][f][d] up weights in wdt for MOE_PATH_DENSE
                                   (moe_materialize_up), else NULL          */
    const void *down_dense;     /* [E+S][d][f] W^down transposed, in wdt, for the
                                   dense path (moe_transpose_down), or NULL.
                                   With it the dense path runs the 256 x 256-tile
                                   MFMA GEMM in bf16 or fp16; without it, bf16
                                   layers only, the older kernels.          */
    float density;              /* expected fraction of the f channels active per
                                   token under the thresholds (e.g. measured
                                   from nnz exports, or 1 - the calibrated
                                   sparsity); <= 0: 0.5.  Read by MOE_PATH_AUTO
                                   and MOE_PATH_MIXED only.                  */
} moe_layer;

/* Optional device outputs of moe_layer_forward (any field may be NULL). */
typedef struct {
    int32_t *topk_idx;          /* [T][k]                                   */
    float *topk_w;              /* [T][k]                                   */
    float *logits;              /* [T][E]                                   */
    int32_t *expert_count;      /* [E] tokens per routed expert             */
    uint8_t *masks;             /* [T][k+S][f] 0/1, sparse path only: slot s<k is
                                   the token's s-th routed expert, slot k+i its
                                   i-th shared expert                        */
    int32_t *eam_row;           /* [E] int32: this call's tokens per routed expert
                                   (the layer's row of the iteration-level EAM)
                                   are ADDED into it, so a row kept across the
                                   calls of a request accumulates the request-
                                   level EAM (MoE-Infinity review, "4.3")     */
    uint64_t *mask_bits;        /* [T][k+S][f/64] the masks of `masks` as bits:
                                   channel 64 i + l at bit l of word i (sparse
                                   path only)                                */
    int32_t *nnz;               /* [T][k+S] active channels per mask (sparse
                                   path only)                                */
    uint8_t *expert_dense;      /* [E]: 1 where the routed expert took the dense
                                   path in this call, else 0 (the shared
                                   experts take it when the call is dense, or
                                   under MOE_PATH_MIXED when T reaches
                                   moe_mixed_dense_min)                      */
} moe_layer_trace;

/*
 * Router: logits = x R^T (+ bias), top-k experts per token with ties going to
 * the lower expert index, weights = softmax over the k chosen logits
 * (renormalize=1) or the full softmax at the chosen experts (renormalize=0);
 * then the T*k (token, slot) pairs grouped by expert
 * (MoE-Infinity review, "A3 背景" and "4.3"; MoE-Lightning review, "MoE 模型架构").
 *   x [T][d] in xdt (f16/bf16/f32), router_w [E][d] in rdt, router_bias [E] or NULL.
 * Outputs:
 *   topk_idx [T][k] int32, topk_w [T][k] fp32,
 *   expert_count [E] int32, expert_offset [E+1] int32 (exclusive prefix),
 *   pair_by_expert [T*k] int32: pairs p = t*k + s of expert e, ascending, at
 *   expert_offset[e] ..; logits_out [T][E] fp32 or NULL.
 * Limits: 1 <= k <= E <= 1024, T*k <= 65536.
 */
moe_status moe_route_topk(const void *x, moe_dtype xdt, int T, int d,
                          const void *router_w, moe_dtype rdt, const float *router_bias,
                          int E, int k, int renormalize,
                          int32_t *topk_idx, float *topk_w,
                          int32_t *expert_count, int32_t *expert_offset,
                          int32_t *pair_by_expert, float *logits_out,
                          void *ws, size_t ws_bytes, void *stream);

/*
 * One compressed expert on T tokens (FloE review, Algorithm 1):
 *   v = x W^up (INT2, fp32 accumulation), mask = |v| > threshold,
 *   h = SiLU(x gate_t[mask]^T) * v[mask], y_t = token_scale_t * h W^down[mask].
 *   x [T][d] in xdt (must equal wdt), y [T][d] in ydt (f16/bf16/f32);
 *   token_scale [T] fp32 or NULL (= 1); accumulate != 0 adds into y.
 * Optional exports (NULL = not wanted):
 *   mask_bits [T][f/64] uint64, 8-byte aligned: the mask of line 2 of
 *             Algorithm 1 as bits, channel 64 i + l at bit l of word i;
 *   nnz_out   [T] int32: active channels per token;
 *   mask_out  [T][f] uint8 0/1: the same mask, one byte per channel;
 *   v_out     [T][f] fp32: v.
 * The bitmask and nnz are formed from the byte mask by one more small kernel
 * (staged in the workspace when mask_out is NULL).
 */
moe_status moe_expert_forward_sparse(const moe_expert_view *e, int d, int f, moe_dtype wdt,
                                     const void *x, moe_dtype xdt, int T,
                                     const float *token_scale, int accumulate,
                                     void *y, moe_dtype ydt,
                                     uint64_t *mask_bits, int32_t *nnz_out,
                                     uint8_t *mask_out, float *v_out,
                                     void *ws, size_t ws_bytes, void *stream);

/*
 * moe_expert_forward_sparse for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, outputs and errors, with no workspace
 * argument.  Its workspace is a static device array of
 * moe_noalloc_scratch_bytes() bytes (32 MiB) that each GPU the library runs on
 * holds until the process ends; the array of the device current on the calling
 * thread is used.  Nothing is allocated and nothing is freed.  Shapes whose
 * workspace (moe_workspace_size(MOE_OP_EXPERT, T, d, f)) exceeds the array
 * return MOE_ERR_UNSUPPORTED (T = 1..8 at d = 4096, f = 14336 fit).  Every call
 * on one GPU shares that GPU's array, which keeps the last call's contents
 * (nothing in it needs to start at zero): calls that overlap on one GPU (other
 * streams, other threads) race and give wrong results; order them on one
 * stream.  MOE_ERR_HIP if the array's device address cannot be found.
 */
moe_status moe_expert_forward_sparse_noalloc(const moe_expert_view *e, int d, int f,
                                             moe_dtype wdt, const void *x, moe_dtype xdt, int T,
                                             const float *token_scale, int accumulate,
                                             void *y, moe_dtype ydt,
                                             uint64_t *mask_bits, int32_t *nnz_out,
                                             uint8_t *mask_out, float *v_out, void *stream);

/* Size in bytes of the static scratch array of moe_expert_forward_sparse_noalloc. */
size_t moe_noalloc_scratch_bytes(void);

/*
 * The same expert with the up projection at 8, 4, 2 or 1 bits per code (FloE
 * review, "敏感度分析": the up projection quantised to INT8/INT4/INT2/INT1).
 * bits == 2 is moe_expert_forward_sparse with the INT2 format above.  For 8, 4
 * and 1: up_q [f][d*bits/8], input k of channel j at bit k*bits of row j
 * (least significant bits first), up_sz [f][d/64][2] as for INT2 with
 * 2^bits - 1 levels (moe_pack_up_bits).  Other arguments, outputs and the
 * mask rule as moe_expert_forward_sparse; the output is bit-reproducible.
 * The same fused kernel runs every width (only the decode of the codes
 * differs).  Limits for 8, 4, 1 bits: d a multiple of 64 from 512 to 4096
 * (else MOE_ERR_UNSUPPORTED); T as for INT2.
 * Workspace: moe_workspace_size(MOE_OP_EXPERT_BITS, T, d, f) bytes (the INT2
 * call's workspace at the same sizes).
 */
moe_status moe_expert_forward_sparse_bits(const moe_expert_view *e, int bits, int d, int f,
                                          moe_dtype wdt, const void *x, moe_dtype xdt, int T,
                                          const float *token_scale, int accumulate,
                                          void *y, moe_dtype ydt,
                                          uint64_t *mask_bits, int32_t *nnz_out,
                                          uint8_t *mask_out, float *v_out,
                                          void *ws, size_t ws_bytes, void *stream);

/*
 * One MoE layer: route (as moe_route_topk) and combine
 *   y_t = sum_s w_{t,s} a_{e(t,s)}(x_t) + sum_i a_{E+i}(x_t)
 * where a_e is Algorithm 1 (MOE_PATH_SPARSE) or the dense SwiGLU with the up
 * weights in L->up_dense (MOE_PATH_DENSE: bf16 or fp16 with L->down_dense; bf16
 * only without it).
 * MOE_PATH_AUTO and MOE_PATH_MIXED choose by one cost model (MoE-Lightning
 * review, "层次化屋顶模型": time = bytes / attainable bandwidth, the expert FFN's
 * operational intensity growing with its tokens).  In units of d f bytes, an
 * expert with n tokens read by the sparse path costs its chunks of at most TB
 * tokens (TB = 1, 2 or 4, as the sparse kernel chunks this call), a chunk of
 * m tokens reading the INT2 up codes and scales (5/16) and the gate and down
 * rows of the union of its tokens' masks (4 u, u = 1 - (1 - L->density)^m);
 * the dense path reads the 16-bit gate, up and down weights once (6).  The
 * dense GEMM streams its weights at about twice the rate of the multi-token
 * sparse kernel, so the dense path is taken when its bytes are under twice
 * the sparse path's.  Both need L->up_dense and L->down_dense (the 256 x
 * 256-tile GEMM) and a call without mask exports; otherwise they take the
 * sparse path, except that bf16 layers with up_dense alone take the older
 * dense kernels for the whole call when T k >= 8 E.
 *   MOE_PATH_AUTO decides per call, on the host, from the expected bytes of
 *   each path with every routed expert receiving each token with probability
 *   k / E (the shared experts all T tokens).  The whole call then takes one
 *   path: serialising a partly filled sparse kernel and partly filled GEMMs
 *   is slower than either path alone on the measured layers.
 *   MOE_PATH_MIXED decides per expert, on the device, from the call's
 *   counts (no host synchronisation): the experts (routed and shared) whose
 *   token count reaches moe_mixed_dense_min take the dense path and the
 *   others the sparse path, in one call.  Its GEMMs run on a library stream
 *   of the current device, forked from `stream` after the routing and joined
 *   back before the reduce by events, so that the sparse kernel and the
 *   GEMMs share the GPU.  That stream (default priority) and its events are
 *   created by the device's first MIXED call and kept until the process
 *   ends; a call made under graph capture before then runs both on `stream`
 *   in order.  The fork and join are serialised across host threads.
 *   x [T][d] in xdt (== L->wdt), y [T][d] in ydt (overwritten).
 * trace (host struct, NULL allowed) receives the optional exports.
 */
moe_status moe_layer_forward(const moe_layer *L, const void *x, moe_dtype xdt, int T,
                             void *y, moe_dtype ydt, moe_path path,
                             const moe_layer_trace *trace,
                             void *ws, size_t ws_bytes, void *stream);

/*
 * MOE_PATH_AUTO's choice for a call of T tokens on this layer (without mask
 * exports, dense weights 16-byte aligned): 1 when the call takes the dense
 * path (every expert with tokens), 0 when it takes the sparse path.  Host
 * arithmetic only; the same value the layer call uses.  0 for invalid
 * arguments.
 */
int moe_auto_dense_min(const moe_layer *L, int T);

/*
 * MOE_PATH_MIXED's per-expert rule for a call of T tokens on this layer: the
 * token count from which an expert takes the dense path (the shared experts
 * take it when T reaches it), or 0 when the call takes the sparse path
 * throughout (no GEMM weights, or no expert can reach the count).  Host
 * arithmetic only; the same value the layer call uses.
 */
int moe_mixed_dense_min(const moe_layer *L, int T);

/*
 * Threshold calibration (FloE review, "高效稀疏 GEMV 内核": t_ij sets the
 * activation sparsity; the pages leave its placement open).  t_out[0] (fp32,
 * device) = the q-quantile of |v| over the n values of v (fp32, device; e.g.
 * the v_out export of moe_expert_forward_sparse on calibration tokens), with
 * linear interpolation between order statistics: h = (n - 1) q,
 * a = |v|_(floor h), b = |v|_(floor h + 1) (both the largest when h >= n - 1),
 * g = h - floor h, t = a + (b - a) g (b - (b - a)(1 - g) when g >= 1/2) in
 * fp64, rounded to fp32 (the interpolation numpy's quantile uses).  The order
 * statistics are found on the GPU by a radix select on the bit patterns of
 * |v|: no host synchronisation.  v must be finite; 1 <= n < 2^31, 0 <= q <= 1.
 * Workspace: moe_workspace_size(MOE_OP_CALIBRATE, ...) bytes (sizes unused).
 */
moe_status moe_calibrate_threshold(const float *v, long long n, double q, float *t_out,
                                   void *ws, size_t ws_bytes, void *stream);

/*
 * Nearest stored request-level EAM (MoE-Infinity review, "4.5": the EAMs are
 * compared flattened, by cosine distance, and the smallest distance is the
 * match; "4.3": an EAM counts the tokens routed to each of the L x E experts).
 *   eamc [n][len] int32 (device): n stored EAMs, each flattened (len = L E);
 *   query [len] int32 (device).
 *   dist_i = 1 - <q, b_i> / sqrt(|q|^2 |b_i|^2), the dot product and squared
 *   norms exact in 64-bit integers, the rest in fp64 (not clipped, so it may be
 *   a rounding step below 0); dist_i = 1 when q or b_i is all zeros.
 *   Entries must lie in [0, 2^22): a stored EAM with an entry outside gets NaN
 *   and is never chosen; a query with one gets NaN everywhere.
 * Outputs: idx_out[0] int32 = the i of the smallest dist_i (the lowest i among
 * equal ones; -1 when every dist_i is NaN); dist_out [n] fp64 or NULL.
 * Limits: 1 <= n, 1 <= len <= 2^17.  Workspace (only when dist_out is NULL):
 * moe_workspace_size(MOE_OP_EAMC, n, len, ...) bytes.
 */
moe_status moe_eamc_match(const int32_t *eamc, int n, int len, const int32_t *query,
                          int32_t *idx_out, double *dist_out,
                          void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes needed by `op` at these sizes (0 when the sizes are invalid). */
size_t moe_workspace_size(moe_op op, int T, int d, int f, int E, int k, int S);

/* Zero-fill a workspace with a kernel (safe inside stream capture). */
moe_status moe_workspace_init(void *ws, size_t ws_bytes, void *stream);

/*
 * Quantise up weights to the INT2 format above (FloE review, "混合压缩策略").
 *   w_up_t [f][d] in dt (f32/f16/bf16), row j = column j of W^up.
 *   Per channel j and group of 64 inputs, in fp32: mn, mx = min, max;
 *   s = fp16_rne((mx - mn) / 3) (1 if that is 0); z = fp16_rne(-mn / s);
 *   q = clamp(round_half_even(w / s + z), 0, 3).
 * Outputs up_q [f][d/4], up_sz [f][d/64][2].  d % 64 == 0, f >= 1.
 * Inputs are expected finite with |w| small enough that (mx - mn) / 3 fits fp16.
 */
moe_status moe_pack_up_int2(const void *w_up_t, moe_dtype dt, int d, int f,
                            uint8_t *up_q, uint16_t *up_sz, void *stream);

/*
 * Quantise up weights to 8, 4, 2 or 1 bits: the scheme of moe_pack_up_int2
 * with L = 2^bits - 1 levels, s = fp16_rne((mx - mn) / L) (1 if 0),
 * q = clamp(round_half_even(w / s + z), 0, L); codes packed plainly (input k at
 * bit k*bits of its row); bits == 2 gives the INT2 format.  Outputs up_q
 * [f][d*bits/8] (16-byte aligned), up_sz [f][d/64][2].  d % 64 == 0, f >= 1.
 */
moe_status moe_pack_up_bits(const void *w_up_t, moe_dtype dt, int d, int f, int bits,
                            uint8_t *up_q, uint16_t *up_sz, void *stream);

/*
 * Dense-path up weights: out[j][k] = rne(s * (q - z)) evaluated exactly, from
 * the INT2 format, rounded to dt (MOE_BF16 or MOE_F16): one-off preparation of
 * moe_layer.up_dense for MOE_PATH_DENSE.  up_q [f][d/4], up_sz [f][d/64][2],
 * out [f][d].  d % 64 == 0.
 */
moe_status moe_materialize_up(const uint8_t *up_q, const uint16_t *up_sz, int d, int f,
                              moe_dtype dt, uint16_t *out, void *stream);

/* moe_materialize_up with dt = MOE_BF16. */
moe_status moe_materialize_up_bf16(const uint8_t *up_q, const uint16_t *up_sz, int d, int f,
                                   uint16_t *out, void *stream);

/*
 * Dense-path down weights (one-off preparation of moe_layer.down_dense): for
 * each of n experts, out [d][f] = the transpose of down [f][d] (16-bit
 * elements, bf16 or fp16 alike), so that the dense down product reads both of
 * its operands along the contracted dimension f.  The sparse path keeps
 * reading `down` row by row (FloE review, "高效稀疏 GEMV 内核": W^down stored
 * transposed so that an active channel's weights are contiguous); the dense
 * path contracts over all channels at once and wants the other order.
 */
moe_status moe_transpose_down(const void *down, int n, int d, int f, void *out, void *stream);

/* Static, human-readable name of a status code. */
const char *moe_status_string(moe_status s);

/* Static string: SHA-256 (64 hex digits) of the sources this binary was built
 * from (every file of csrc/ and this header, in name order), so that a binding
 * can refuse a library that is older than its sources. */
const char *moe_build_sources_sha256(void);

#ifdef __cplusplus
}
#endif

#endif /* MOEFFN_H */
