// C ABI of libmoeffn: argument validation, workspace layout and dispatch.
// Every check runs on the host before anything is enqueued; no HIP call is made
// for an invalid request, so the error paths can be exercised without a GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <new>

#include "../../include/moeffn.h"
#include "internal.hpp"

using namespace moeffn;

namespace {

constexpr size_t kAlign = 256;
constexpr int kEamcMaxLen = 1 << 17;         // entries of one flattened EAM

size_t up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

bool aligned(const void *p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool is16(moe_dtype t) { return t == MOE_F16 || t == MOE_BF16; }

bool valid_out(moe_dtype t) { return t == MOE_F16 || t == MOE_BF16 || t == MOE_F32; }

// Hidden sizes of the INT2 sparse path: whole groups of 64 inputs, up to the
// widest kernel geometry (256 groups).
bool supported_d(int d)
{
    return d >= 64 && d <= 16384 && d % 64 == 0;
}

int pow2ceil(int v)
{
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

// Work split of the sparse kernel: about 256 workgroups over all expert slots
// (one per compute unit), channels per tile a multiple of 8 and at most 1024,
// and the fp32 partial rows (rows x tiles x d) kept under 256 MiB.
struct TilePlan {
    int cpw, tiles;
};

TilePlan plan_tiles(int f, int slots, long long rows, int d)
{
    const int fr = (f + 7) / 8 * 8;
    int tiles = (256 + slots - 1) / slots;
    int cpw = (f + tiles - 1) / tiles;
    cpw = (cpw + 7) / 8 * 8;
    if (cpw < 8) cpw = 8;
    if (cpw > 1024) cpw = 1024;
    const long long cap = 256ll << 20;
    for (;;) {
        tiles = (f + cpw - 1) / cpw;
        if (rows * tiles * d * 4 <= cap || cpw >= fr || cpw >= 1024) break;
        cpw = cpw * 2 > 1024 ? 1024 : cpw * 2;
    }
    if (cpw > fr) cpw = fr;
    tiles = (f + cpw - 1) / cpw;
    return {cpw, tiles};
}

// Tokens per chunk of the sparse kernel for about `n` tokens per expert: at
// most 4 up to d = 4096, 2 up to 8192 and 1 beyond (larger chunks need more
// registers than the kernel has).
int choose_tb(long long n, int d)
{
    int tb = 1;
    while (tb < n && tb < 4) tb <<= 1;
    const int tbmax = d <= 4096 ? 4 : (d <= 8192 ? 2 : 1);
    return tb > tbmax ? tbmax : tb;
}

// Grid of the sparse kernel: token chunks x tiles of channels.
struct SparsePlan {
    int tb;         // tokens per chunk
    int slots;      // chunk slots (an upper bound in a layer: routed chunks are data-dependent)
    TilePlan tp;
};

// (At most about 60 KB of LDS for every supported d, tb and cpw <= 1024.)
SparsePlan expert_plan(int T, int d, int f)
{
    const int tb = choose_tb(T, d);
    const int slots = (T + tb - 1) / tb;
    return SparsePlan{tb, slots, plan_tiles(f, slots, T, d)};
}

// Layer: chunks sized for the average number of tokens a routed expert
// receives.  The A experts that receive n_e tokens (sum n_e = T k) hold
// sum ceil(n_e / tb) <= (T k + A (tb - 1)) / tb chunks, A <= min(E, T k); the
// S shared experts hold ceil(T / tb) chunks each.  The grid covers that bound;
// the tiles per chunk are sized for the expected count (half a chunk of
// padding per expert), so that the chunks that do exist fill the chip.
SparsePlan layer_plan(int T, int d, int f, int E, int k, int S)
{
    const long long tk = (long long)T * k;
    const int tb = choose_tb((tk + E - 1) / E, d);
    const long long act = E < tk ? E : tk;
    const long long shared = (long long)S * ((T + tb - 1) / tb);
    const long long bound = shared + (tk + act * (tb - 1)) / tb;
    const long long expect = shared + (2 * tk + act * (tb - 1) + 2 * tb - 1) / (2 * tb);
    return SparsePlan{tb, (int)bound, plan_tiles(f, (int)expect, (long long)T * (k + S), d)};
}

size_t expert_ws_core(int T, int d, int f)
{
    const TilePlan tp = expert_plan(T, d, f).tp;
    return up((size_t)T * tp.tiles * d * 4);
}

size_t expert_ws_bytes(int T, int d, int f) { return expert_ws_core(T, d, f) + up((size_t)T * f); }

struct LayerWs {
    int32_t *topk_idx;
    float *topk_w;
    int32_t *count, *offset, *pairs, *active, *n_active;
    int32_t *chunk_tab, *n_chunks;
    float *part;
    float *h;
    float *lg;              // [T][E] router logits (wide-router split)
    int32_t *chunk_rec;     // [T*k][4] single-token chunk records
    uint8_t *masks;         // [T][k+S][f] byte masks staged for the bitmask / nnz exports
    int32_t *chunk_tab2, *n_chunks2;    // dense chunks
    uint8_t *expert_dense;  // [E] path of each routed expert
};

size_t layer_ws_bytes(int T, int d, int f, int E, int k, int S, LayerWs *out, void *base)
{
    const long long rows = (long long)T * (k + S);
    const TilePlan tp = layer_plan(T, d, f, E, k, S).tp;
    const size_t part_tiles = (size_t)(tp.tiles > kDenseKSplit ? tp.tiles : kDenseKSplit);
    size_t o = 0;
    size_t off[18];
    off[0] = o; o += up(4);
    off[1] = o; o += up((size_t)T * k * 4);
    off[2] = o; o += up((size_t)T * k * 4);
    off[3] = o; o += up((size_t)E * 4);
    off[4] = o; o += up((size_t)(E + 1) * 4);
    off[5] = o; o += up((size_t)T * k * 4);
    off[6] = o; o += up((size_t)E * 4);
    off[7] = o; o += up(4);
    off[8] = o; o += up((size_t)rows * part_tiles * d * 4);
    off[9] = o; o += up(dense_h_bytes(T, f, k, S));
    off[10] = o; o += up((size_t)T * k * 4);           // every chunk holds at least one pair
    off[11] = o; o += up(4);
    off[12] = o; o += up((size_t)T * E * 4);
    off[13] = o; o += up((size_t)T * k * 16);
    off[14] = o; o += up((size_t)rows * f);
    off[15] = o; o += up((size_t)T * k * 4);           // dense chunks (at most one per pair)
    off[16] = o; o += up(4);
    off[17] = o; o += up((size_t)E);
    if (out) {
        char *p = (char *)base;
        out->topk_idx = (int32_t *)(p + off[1]);
        out->topk_w = (float *)(p + off[2]);
        out->count = (int32_t *)(p + off[3]);
        out->offset = (int32_t *)(p + off[4]);
        out->pairs = (int32_t *)(p + off[5]);
        out->active = (int32_t *)(p + off[6]);
        out->n_active = (int32_t *)(p + off[7]);
        out->part = (float *)(p + off[8]);
        out->h = (float *)(p + off[9]);
        out->chunk_tab = (int32_t *)(p + off[10]);
        out->n_chunks = (int32_t *)(p + off[11]);
        out->lg = (float *)(p + off[12]);
        out->chunk_rec = (int32_t *)(p + off[13]);
        out->masks = (uint8_t *)(p + off[14]);
        out->chunk_tab2 = (int32_t *)(p + off[15]);
        out->n_chunks2 = (int32_t *)(p + off[16]);
        out->expert_dense = (uint8_t *)(p + off[17]);
    }
    return o;
}

// ---- scratch of the allocation-free entry point ------------------------------
// A file-scope device array serves as the workspace of
// moe_expert_forward_sparse_noalloc.  Each GPU holds its own copy at its own
// address, looked up once per device with hipGetSymbolAddress; host code uses
// only that address (the array's name is a host-side stand-in, not a device
// pointer).  Every call on one GPU shares its copy.
constexpr size_t kScratchBytes = 32u << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The scratch address on the calling thread's current device (null on error).
void *scratch_for_current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

// ---- second stream of mixed layer calls ------------------------------------
// A call that runs both the sparse kernel and the GEMMs (MOE_PATH_MIXED)
// launches the GEMMs on a library stream of the caller's device, forked from
// and joined back into the caller's stream by events.  The two kernel
// families write disjoint partial rows, so they can share the compute units
// instead of each running partly filled.  The stream (default priority) and
// the events are created by the device's first such call; a call under graph
// capture that finds none runs both in order on the caller's stream.  The
// fork, the launches on the library stream and the join are made under one
// lock, so that concurrent calls from several host threads keep their own
// dependencies.
struct ForkState {
    hipStream_t s2 = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_fork_mu;
ForkState g_fork[kMaxDevices];

// The current device's fork state (g_fork_mu held), or null: creation failed,
// or it does not exist yet and `s` is capturing.
ForkState *fork_state(hipStream_t s)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    ForkState &fs = g_fork[dev];
    if (fs.s2) return &fs;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
    hipStream_t s2 = nullptr;
    hipEvent_t e1 = nullptr, e2 = nullptr;
    if (hipStreamCreateWithFlags(&s2, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&e1, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&e2, hipEventDisableTiming) != hipSuccess) {
        if (e1) (void)hipEventDestroy(e1);
        (void)hipStreamDestroy(s2);
        return nullptr;
    }
    fs.s2 = s2;
    fs.fork = e1;
    fs.join = e2;
    return &fs;
}

// Split of f in the dense down product: enough workgroups (d / 256 column
// tiles per chunk of tokens) for about two per compute unit, at most 4 (the
// partial-row region holds 4 slices per row), each slice a multiple of 64.
// Token rows per dense chunk and tile, from the routed experts' average
// token count: up to 32, 64 rows (two workgroups per compute unit); up to 96,
// 128 rows (three stages, two blocks in flight); else 256.  The weight stream
// and its latency bound the smaller cases.  Near 64 tokens on average many
// experts would spill into a second, nearly empty 64-row chunk that streams
// the weights again, hence the margins.
int gemm_tile_rows(int T, int k, int E)
{
    const long long tk = (long long)T * k;
    if (tk <= 32ll * E) return 64;
    if (tk <= 96ll * E) return 128;
    return kGemmChunk;
}

int gemm_ksplit(int T, int k, int E, int S, int d, int f, int mt)
{
    const long long tk = (long long)T * k;
    const long long act = E < tk ? E : tk;
    const long long expect = (long long)S * ((T + mt - 1) / mt) + (tk + mt - 1) / mt + act / 2;
    int ks = 1;
    while (ks < kDenseKSplit && expect * (d / 256) * ks < 512 && f % (64 * ks * 2) == 0) ks *= 2;
    return ks;
}

// Cost model of MOE_PATH_AUTO and MOE_PATH_MIXED (MoE-Lightning review,
// "层次化屋顶模型": time = bytes moved / attainable bandwidth, the expert FFN's
// operational intensity growing with its tokens).  Bytes in units of d f:
// the sparse path reads, per chunk of m <= tb tokens of one expert, the INT2
// codes and scales (5/16) and the gate and down rows of the union of the m
// masks (4 u, u = 1 - (1 - density)^m); the dense path reads the three 16-bit
// matrices once (6).  The dense GEMM streams its weights at about twice the
// rate at which the multi-token sparse kernel streams codes and rows (4-6
// against 2-3 TB/s on MI355X), so dense wins when its bytes are under twice
// the sparse bytes.
constexpr double kDenseBytes = 6.0;
constexpr double kDenseOverSparseRate = 2.0;

struct PathCost {
    int tb;                 // 1, 2 or 4
    double ch[5];           // a chunk of m tokens
    PathCost(int tb_, float density) : tb(tb_)
    {
        const double rho = density > 0.f && density <= 1.f ? (double)density : 0.5;
        ch[0] = 0.0;
        for (int m = 1; m <= 4; ++m) ch[m] = 0.3125 + 4.0 * (1.0 - std::pow(1.0 - rho, (double)m));
    }
    // one expert with n tokens on the sparse path
    double sparse(long long n) const { return (double)(n / tb) * ch[tb] + ch[n % tb]; }
    bool dense_wins(double dense_bytes, double sparse_bytes) const
    {
        return dense_bytes < kDenseOverSparseRate * sparse_bytes;
    }
};

// MOE_PATH_MIXED, per expert: the smallest token count n whose sparse chunks
// take longer than reading the dense weights once.
int dense_min_tokens(int tb, float density)
{
    const PathCost c(tb, density);
    int n = 1;
    while (!c.dense_wins(kDenseBytes, c.sparse(n))) ++n;    // sparse(n) grows by >= 5/16 per chunk
    return n;
}

// E[g(n)] for n ~ Binomial(T, p), 0 < p < 1: outward from the mode, where the
// probability is at least about 1 / (2.5 sqrt(T p (1 - p)) + 1), until the
// terms are negligible.
template <class G>
double binomial_mean(int T, double p, G g)
{
    const int n0 = (int)std::floor((T + 1) * p) > T ? T : (int)std::floor((T + 1) * p);
    const double r = p / (1.0 - p);
    const double p0 = std::exp(std::lgamma(T + 1.0) - std::lgamma(n0 + 1.0) - std::lgamma(T - n0 + 1.0) +
                               n0 * std::log(p) + (T - n0) * std::log1p(-p));
    double s = p0 * g(n0), q = p0;
    for (int n = n0; n < T && q > 1e-18; ++n) {
        q *= (double)(T - n) / (n + 1) * r;
        s += q * g(n + 1);
    }
    q = p0;
    for (int n = n0; n > 0 && q > 1e-18; --n) {
        q *= (double)n / (T - n + 1) / r;
        s += q * g(n - 1);
    }
    return s;
}

// MOE_PATH_AUTO, per call: the expected bytes of the whole call on each path,
// with every routed expert receiving each token with probability k / E
// (uniform routing; the call's counts are known only on the device) and the
// shared experts all T tokens.
bool auto_takes_dense(int T, int E, int k, int S, int tb, float density)
{
    const PathCost c(tb, density);
    double sparse = S * c.sparse(T), dense = S * kDenseBytes;
    if (k >= E) {
        sparse += E * c.sparse(T);
        dense += E * kDenseBytes;
    } else {
        const double p = (double)k / E;
        sparse += E * binomial_mean(T, p, [&](int n) { return c.sparse(n); });
        dense += E * kDenseBytes * -std::expm1(T * std::log1p(-p));     // P(n > 0)
    }
    return c.dense_wins(dense, sparse);
}

hipError_t launch_sparse(const SparseArgs &a, bool bf16, int tb, hipStream_t s)
{
    return bf16 ? launch_sparse_expert_bf16(a, tb, s) : launch_sparse_expert_f16(a, tb, s);
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

moe_status check_route_args(const void *x, moe_dtype xdt, int T, int d, const void *rw,
                            moe_dtype rdt, int E, int k)
{
    if (!x || !rw) return MOE_ERR_INVALID_ARG;
    if (T < 1 || d < 8 || E < 1 || E > 1024 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
    if (d % 8 != 0) return MOE_ERR_UNSUPPORTED;         // rows are read in 16-byte units
    if ((long long)T * k > 65536) return MOE_ERR_UNSUPPORTED;
    if (!valid_out(xdt) || !valid_out(rdt)) return MOE_ERR_UNSUPPORTED;
    if ((size_t)d * 4 + (size_t)E * 8 + (size_t)k * 8 + 32 > 160 * 1024) return MOE_ERR_UNSUPPORTED;
    if (!aligned(x, xdt == MOE_F32 ? 4 : 2) || !aligned(rw, rdt == MOE_F32 ? 4 : 2))
        return MOE_ERR_ALIGNMENT;
    return MOE_OK;
}

moe_status check_expert_shape(int d, int f, moe_dtype wdt, moe_dtype xdt, int T, moe_dtype ydt)
{
    if (T < 1 || T > 65536 || d < 1 || f < 1) return MOE_ERR_INVALID_ARG;
    if (f % 64 != 0) return MOE_ERR_INVALID_ARG;
    if (!supported_d(d)) return MOE_ERR_UNSUPPORTED;
    if (!is16(wdt) || xdt != wdt || !valid_out(ydt)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

moe_status check_weight_ptrs(const uint8_t *q, const uint16_t *sz, const void *g, const void *dn)
{
    if (!q || !sz || !g || !dn) return MOE_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(g, 16) || !aligned(dn, 16) || !aligned(sz, 4))
        return MOE_ERR_ALIGNMENT;
    return MOE_OK;
}

// The dense kernels a layer can run: the 256 x 256-tile GEMM (bf16 or fp16,
// needs the transposed down weights) or the older bf16 kernels (row-major down).
bool layer_gemm_ok(const moe_layer *L)
{
    return L->up_dense && L->down_dense && L->d % 256 == 0 && L->f % 128 == 0;
}
bool layer_old_ok(const moe_layer *L)
{
    return L->wdt == MOE_BF16 && L->up_dense && L->f % 256 == 0 && L->d % 128 == 0;
}
bool layer_args_ok(const moe_layer *L, int T)
{
    return L && T >= 1 && L->n_routed >= 1 && L->top_k >= 1 && L->top_k <= L->n_routed &&
           L->n_shared >= 0 && L->d > 0 && L->f > 0;
}

// MOE_PATH_AUTO for T tokens: the GEMM layers by the expected-time rule, the
// older bf16 kernels from T k >= 8 E (they serve whole calls only)
bool auto_dense(const moe_layer *L, int T)
{
    if (layer_gemm_ok(L)) {
        const SparsePlan sp = layer_plan(T, L->d, L->f, L->n_routed, L->top_k, L->n_shared);
        return auto_takes_dense(T, L->n_routed, L->top_k, L->n_shared, sp.tb, L->density);
    }
    return layer_old_ok(L) && (long long)T * L->top_k >= 8ll * L->n_routed;
}

// MOE_PATH_MIXED for T tokens: the per-expert token threshold, or 0 when no
// expert can reach it (or the layer has no GEMM weights)
int mixed_dense_min(const moe_layer *L, int T)
{
    if (!layer_gemm_ok(L)) return 0;
    const SparsePlan sp = layer_plan(T, L->d, L->f, L->n_routed, L->top_k, L->n_shared);
    const int n = dense_min_tokens(sp.tb, L->density);
    return n > T ? 0 : n;
}

}  // namespace

extern "C" {

#ifndef MOE_SOURCES_SHA256
#define MOE_SOURCES_SHA256 "unknown"
#endif

const char *moe_build_sources_sha256(void) { return MOE_SOURCES_SHA256; }

const char *moe_status_string(moe_status s)
{
    switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MOE_ERR_ALIGNMENT: return "misaligned pointer";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

size_t moe_workspace_size(moe_op op, int T, int d, int f, int E, int k, int S)
{
    if (T < 1 || d < 1) return 0;
    switch (op) {
    case MOE_OP_EXPERT: return f < 1 ? 0 : expert_ws_bytes(T, d, f);
    case MOE_OP_ROUTE:
        if (E < 1) return 0;
        return up(4) + up((size_t)T * E * 4);          // logits of the wide-router split
    case MOE_OP_LAYER:
        if (E < 1 || k < 1 || k > E || S < 0 || f < 1) return 0;
        return layer_ws_bytes(T, d, f, E, k, S, nullptr, nullptr);
    case MOE_OP_CALIBRATE:
        return up(calibrate_ws_bytes());
    case MOE_OP_EXPERT_BITS:
        return f < 1 ? 0 : expert_ws_bytes(T, d, f);
    case MOE_OP_EAMC:
        return d > kEamcMaxLen ? 0 : up((size_t)T * 8);   // T stored EAMs of d entries
    }
    return 0;
}

moe_status moe_eamc_match(const int32_t *eamc, int n, int len, const int32_t *query,
                          int32_t *idx_out, double *dist_out, void *ws, size_t ws_bytes,
                          void *stream)
{
    if (!eamc || !query || !idx_out || n < 1 || len < 1 || len > kEamcMaxLen)
        return MOE_ERR_INVALID_ARG;
    if (!aligned(eamc, 4) || !aligned(query, 4) || !aligned(idx_out, 4) ||
        (dist_out && !aligned(dist_out, 8)))
        return MOE_ERR_ALIGNMENT;
    double *dist = dist_out;
    if (!dist) {
        if (!ws || ws_bytes < moe_workspace_size(MOE_OP_EAMC, n, len, 0, 0, 0, 0))
            return MOE_ERR_WORKSPACE;
        if (!aligned(ws, 16)) return MOE_ERR_ALIGNMENT;
        dist = (double *)ws;
    }
    return hip_status(launch_eamc_match(eamc, n, len, query, idx_out, dist, (hipStream_t)stream));
}

moe_status moe_calibrate_threshold(const float *v, long long n, double q, float *t_out,
                                   void *ws, size_t ws_bytes, void *stream)
{
    if (!v || !t_out || n < 1 || n >= (1ll << 31) || !(q >= 0.0 && q <= 1.0))
        return MOE_ERR_INVALID_ARG;
    if (!aligned(v, 4) || !aligned(t_out, 4)) return MOE_ERR_ALIGNMENT;
    if (!ws || ws_bytes < up(calibrate_ws_bytes())) return MOE_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return MOE_ERR_ALIGNMENT;
    // virtual index and neighbours as numpy's linear quantile forms them
    const double h = (double)(n - 1) * q;
    long long lo = (long long)std::floor(h), hi = lo + 1;
    const double gamma = h - std::floor(h);
    if (h >= (double)(n - 1)) lo = hi = n - 1;
    if (h < 0.0) lo = hi = 0;
    return hip_status(launch_calibrate(v, n, lo, hi, gamma, t_out, ws, (hipStream_t)stream));
}

moe_status moe_workspace_init(void *ws, size_t ws_bytes, void *stream)
{
    if (!ws || ws_bytes == 0) return MOE_ERR_INVALID_ARG;
    if (!aligned(ws, 4) || ws_bytes % 4 != 0) return MOE_ERR_ALIGNMENT;
    return hip_status(launch_fill_zero(ws, ws_bytes, (hipStream_t)stream));
}

int moe_auto_dense_min(const moe_layer *L, int T)
{
    if (!layer_args_ok(L, T)) return 0;
    return auto_dense(L, T) ? 1 : 0;
}

int moe_mixed_dense_min(const moe_layer *L, int T)
{
    if (!layer_args_ok(L, T)) return 0;
    return mixed_dense_min(L, T);
}

moe_status moe_route_topk(const void *x, moe_dtype xdt, int T, int d, const void *router_w,
                          moe_dtype rdt, const float *router_bias, int E, int k, int renormalize,
                          int32_t *topk_idx, float *topk_w, int32_t *expert_count,
                          int32_t *expert_offset, int32_t *pair_by_expert, float *logits_out,
                          void *ws, size_t ws_bytes, void *stream)
{
    moe_status st = check_route_args(x, xdt, T, d, router_w, rdt, E, k);
    if (st != MOE_OK) return st;
    if (!topk_idx || !topk_w || !expert_count || !expert_offset || !pair_by_expert)
        return MOE_ERR_INVALID_ARG;
    if (!ws || ws_bytes < moe_workspace_size(MOE_OP_ROUTE, T, d, 0, E, k, 0))
        return MOE_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return MOE_ERR_ALIGNMENT;
    RouteArgs a{};
    a.x = x; a.xdt = xdt; a.T = T; a.d = d;
    a.rw = router_w; a.rdt = rdt; a.bias = router_bias;
    a.E = E; a.k = k; a.renorm = renormalize ? 1 : 0;
    a.topk_idx = topk_idx; a.topk_w = topk_w; a.logits = logits_out;
    a.count = expert_count; a.offset = expert_offset; a.pairs = pair_by_expert;
    a.active = nullptr; a.n_active = nullptr;
    a.lg_buf = route_split(d, E, rdt) ? (float *)((char *)ws + up(4)) : nullptr;
    return hip_status(launch_route(a, (hipStream_t)stream));
}

namespace {
// One expert over T tokens with the up codes at `bits` (2: the INT2 format,
// 8 / 4 / 1: plain packing, d = 512 ... 4096): the fused kernel, the reduce,
// and the bitmask / nnz exports when asked for.
static moe_status expert_forward(const moe_expert_view *e, int bits, int d, int f, moe_dtype wdt,
                          const void *x, moe_dtype xdt, int T, const float *token_scale,
                          int accumulate, void *y, moe_dtype ydt, uint64_t *mask_bits,
                          int32_t *nnz_out, uint8_t *mask_out, float *v_out, void *ws,
                          size_t ws_bytes, void *stream)
{
    if (!e || !x || !y) return MOE_ERR_INVALID_ARG;
    moe_status st = check_expert_shape(d, f, wdt, xdt, T, ydt);
    if (st != MOE_OK) return st;
    if (bits != 2 && (d < 512 || d > 4096 || d % 64 != 0)) return MOE_ERR_UNSUPPORTED;
    st = check_weight_ptrs(e->up_q, e->up_sz, e->gate_t, e->down);
    if (st != MOE_OK) return st;
    if (!aligned(x, 16) || !aligned(y, ydt == MOE_F32 ? 4 : 2) ||
        (token_scale && !aligned(token_scale, 4)) || (v_out && !aligned(v_out, 4)) ||
        (mask_bits && !aligned(mask_bits, 8)) || (nnz_out && !aligned(nnz_out, 4)))
        return MOE_ERR_ALIGNMENT;
    if (!ws || ws_bytes < expert_ws_bytes(T, d, f)) return MOE_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return MOE_ERR_ALIGNMENT;

    hipStream_t s = (hipStream_t)stream;
    const bool want_bits = mask_bits || nnz_out;
    if (want_bits && !mask_out) mask_out = (uint8_t *)ws + expert_ws_core(T, d, f);
    const SparsePlan sp = expert_plan(T, d, f);
    const TilePlan tp = sp.tp;
    SparseArgs a{};
    a.d = d; a.f = f;
    a.slots = sp.slots;
    a.cpw = tp.cpw;
    a.tiles = tp.tiles;
    a.up_q = e->up_q; a.up_sz = e->up_sz;
    a.gate = (const uint16_t *)e->gate_t; a.down = (const uint16_t *)e->down;
    a.q_stride = 0; a.sz_stride = 0; a.w_stride = 0;
    a.thr_dev = nullptr; a.thr = e->threshold;
    a.x = (const uint16_t *)x; a.T = T;
    a.token_scale = token_scale;
    a.layer = 0;
    a.part = (float *)ws;
    a.mask_out = mask_out; a.v_out = v_out;
    hipError_t he = bits == 2 ? launch_sparse(a, wdt == MOE_BF16, sp.tb, s)
                              : launch_sparse_expert_bits(a, bits, wdt == MOE_BF16, sp.tb, s);
    if (he != hipSuccess) return MOE_ERR_HIP;
    ReduceArgs r{};
    r.part = a.part; r.tiles = tp.tiles; r.d = d; r.T = T;
    r.layer = 0; r.rows_per_tok = 1; r.k = 1; r.S = 0;
    r.y = y; r.ydt = (int)ydt; r.accumulate = accumulate ? 1 : 0;
    he = launch_reduce(r, s);
    if (he == hipSuccess && want_bits) he = launch_mask_bits(mask_out, T, f, mask_bits, nnz_out, s);
    return hip_status(he);
}
}  // namespace

moe_status moe_expert_forward_sparse(const moe_expert_view *e, int d, int f, moe_dtype wdt,
                                     const void *x, moe_dtype xdt, int T,
                                     const float *token_scale, int accumulate, void *y,
                                     moe_dtype ydt, uint64_t *mask_bits, int32_t *nnz_out,
                                     uint8_t *mask_out, float *v_out, void *ws,
                                     size_t ws_bytes, void *stream)
{
    return expert_forward(e, 2, d, f, wdt, x, xdt, T, token_scale, accumulate, y, ydt, mask_bits,
                          nnz_out, mask_out, v_out, ws, ws_bytes, stream);
}

size_t moe_noalloc_scratch_bytes(void) { return kScratchBytes; }

moe_status moe_expert_forward_sparse_noalloc(const moe_expert_view *e, int d, int f,
                                             moe_dtype wdt, const void *x, moe_dtype xdt, int T,
                                             const float *token_scale, int accumulate, void *y,
                                             moe_dtype ydt, uint64_t *mask_bits, int32_t *nnz_out,
                                             uint8_t *mask_out, float *v_out, void *stream)
{
    if (!e || !x || !y) return MOE_ERR_INVALID_ARG;
    moe_status st = check_expert_shape(d, f, wdt, xdt, T, ydt);
    if (st != MOE_OK) return st;
    if (expert_ws_bytes(T, d, f) > kScratchBytes) return MOE_ERR_UNSUPPORTED;
    void *ws = scratch_for_current_device();
    if (!ws) return MOE_ERR_HIP;
    return moe_expert_forward_sparse(e, d, f, wdt, x, xdt, T, token_scale, accumulate, y, ydt,
                                     mask_bits, nnz_out, mask_out, v_out, ws, kScratchBytes,
                                     stream);
}

moe_status moe_expert_forward_sparse_bits(const moe_expert_view *e, int bits, int d, int f,
                                          moe_dtype wdt, const void *x, moe_dtype xdt, int T,
                                          const float *token_scale, int accumulate, void *y,
                                          moe_dtype ydt, uint64_t *mask_bits, int32_t *nnz_out,
                                          uint8_t *mask_out, float *v_out,
                                          void *ws, size_t ws_bytes, void *stream)
{
    if (bits != 1 && bits != 2 && bits != 4 && bits != 8) return MOE_ERR_INVALID_ARG;
    return expert_forward(e, bits, d, f, wdt, x, xdt, T, token_scale, accumulate, y, ydt,
                          mask_bits, nnz_out, mask_out, v_out, ws, ws_bytes, stream);
}

moe_status moe_layer_forward(const moe_layer *L, const void *x, moe_dtype xdt, int T, void *y,
                             moe_dtype ydt, moe_path path, const moe_layer_trace *trace, void *ws,
                             size_t ws_bytes, void *stream)
{
    if (!L || !x || !y) return MOE_ERR_INVALID_ARG;
    const int d = L->d, f = L->f, E = L->n_routed, S = L->n_shared, k = L->top_k;
    if (S < 0) return MOE_ERR_INVALID_ARG;
    if (k + S > kMaxExpertsPerToken) return MOE_ERR_UNSUPPORTED;
    moe_status st = check_route_args(x, xdt, T, d, L->router_w, L->rdt, E, k);
    if (st != MOE_OK) return st;
    st = check_expert_shape(d, f, L->wdt, xdt, T, ydt);
    if (st != MOE_OK) return st;
    st = check_weight_ptrs(L->up_q, L->up_sz, L->gate_t, L->down);
    if (st != MOE_OK) return st;
    if (!L->thresholds) return MOE_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(y, ydt == MOE_F32 ? 4 : 2) || !aligned(L->thresholds, 4))
        return MOE_ERR_ALIGNMENT;
    if (path != MOE_PATH_SPARSE && path != MOE_PATH_DENSE && path != MOE_PATH_AUTO &&
        path != MOE_PATH_MIXED)
        return MOE_ERR_INVALID_ARG;
    // dense kernels: the 256 x 256-tile GEMM (bf16 or fp16; needs the
    // transposed down weights) or the older bf16 kernels (row-major down)
    const bool want_masks = trace && (trace->masks || trace->mask_bits || trace->nnz);
    const bool gemm_ok = layer_gemm_ok(L);
    const bool old_ok = layer_old_ok(L);
    const SparsePlan sp = layer_plan(T, d, f, E, k, S);
    const bool dense_aligned = L->up_dense && aligned(L->up_dense, 16) &&
                               (!L->down_dense || aligned(L->down_dense, 16));
    int nstar = 0;                  // per expert: experts with >= nstar tokens take the dense path
    if (path == MOE_PATH_MIXED && gemm_ok && dense_aligned && !want_masks) {
        nstar = mixed_dense_min(L, T);              // 0: no expert can reach it
        path = nstar > 0 ? MOE_PATH_DENSE : MOE_PATH_SPARSE;
    } else if (path == MOE_PATH_AUTO || path == MOE_PATH_MIXED) {
        path = dense_aligned && !want_masks && auto_dense(L, T) ? MOE_PATH_DENSE : MOE_PATH_SPARSE;
    }
    const bool mixed = nstar > 1;   // (nstar == 1: every expert with tokens is dense)
    if (path == MOE_PATH_DENSE) {
        if (!gemm_ok && !old_ok) return MOE_ERR_UNSUPPORTED;
        if (!aligned(L->up_dense, 16) || (L->down_dense && !aligned(L->down_dense, 16)))
            return MOE_ERR_ALIGNMENT;
        if (want_masks) return MOE_ERR_UNSUPPORTED;
    }
    if (trace && ((trace->mask_bits && !aligned(trace->mask_bits, 8)) ||
                  (trace->nnz && !aligned(trace->nnz, 4))))
        return MOE_ERR_ALIGNMENT;
    if (!ws || ws_bytes < layer_ws_bytes(T, d, f, E, k, S, nullptr, nullptr))
        return MOE_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return MOE_ERR_ALIGNMENT;

    hipStream_t s = (hipStream_t)stream;
    LayerWs w;
    layer_ws_bytes(T, d, f, E, k, S, &w, ws);

    RouteArgs r{};
    r.x = x; r.xdt = xdt; r.T = T; r.d = d;
    r.rw = L->router_w; r.rdt = L->rdt; r.bias = L->router_bias;
    r.E = E; r.k = k; r.renorm = L->renormalize ? 1 : 0;
    r.topk_idx = (trace && trace->topk_idx) ? trace->topk_idx : w.topk_idx;
    r.topk_w = (trace && trace->topk_w) ? trace->topk_w : w.topk_w;
    r.logits = trace ? trace->logits : nullptr;
    r.count = (trace && trace->expert_count) ? trace->expert_count : w.count;
    r.eam_row = trace ? trace->eam_row : nullptr;
    r.offset = w.offset; r.pairs = w.pairs;
    r.active = w.active; r.n_active = w.n_active;
    r.lg_buf = route_split(d, E, L->rdt) ? w.lg : nullptr;
    const bool use_gemm = path == MOE_PATH_DENSE && gemm_ok;
    if (path == MOE_PATH_SPARSE || mixed) {
        r.chunk = sp.tb; r.chunk_tab = w.chunk_tab; r.n_chunks = w.n_chunks;
        if (sp.tb == 1 && !mixed) r.chunk_rec = w.chunk_rec;
    }
    if (path == MOE_PATH_DENSE) {
        // experts with at least dense_min pairs are listed in 256-token chunks
        r.dense_min = mixed ? nstar : 1;
        r.dense_chunk = gemm_tile_rows(T, k, E); r.chunk_tab2 = w.chunk_tab2; r.n_chunks2 = w.n_chunks2;
    }
    r.expert_dense = (trace && trace->expert_dense) ? trace->expert_dense
                   : (mixed ? w.expert_dense : nullptr);
    const bool shared_dense = path == MOE_PATH_DENSE && (!mixed || T >= nstar);
    // A single token on the sparse path is routed inside the expert kernel:
    // each routed workgroup ranks the logits itself (formed there for routers
    // up to kInlineRouterBytes, else by the logits kernel first), so neither
    // the ranking nor the grouping kernel runs.
    const bool inline_route = path == MOE_PATH_SPARSE && !mixed && T == 1 && sp.tb == 1;
    const size_t router_bytes = (size_t)E * d * (L->rdt == MOE_F32 ? 4 : 2);
    const bool inline_logits_kernel =
        inline_route && (route_split(d, E, L->rdt) || router_bytes > kInlineRouterBytes);
    hipError_t he = hipSuccess;
    if (inline_route) {
        // no grouping kernel writes the per-expert path flags: all sparse
        if (trace && trace->expert_dense) he = launch_fill_u8(trace->expert_dense, (size_t)E, 0, s);
        if (he == hipSuccess && inline_logits_kernel) {
            r.lg_buf = w.lg;
            he = launch_route_logits(r, s);
        }
    } else {
        he = launch_route(r, s);
    }
    if (he != hipSuccess) return MOE_ERR_HIP;

    const size_t qs = (size_t)f * (d / 4), szs = (size_t)f * (d / 64) * 2, wst = (size_t)f * d;
    ReduceArgs red{};
    red.d = d; red.T = T; red.layer = 1; red.rows_per_tok = k + S; red.k = k; red.S = S;
    red.part = w.part;
    red.y = y; red.ydt = (int)ydt; red.accumulate = 0;
    const int mt = gemm_tile_rows(T, k, E);
    const int ksplit = use_gemm ? gemm_ksplit(T, k, E, S, d, f, mt) : 0;
    TilePlan tp = sp.tp;
    if (mixed) {
        // The sparse kernel sees only experts below n* tokens (at most
        // ceil((n* - 1) / tb) chunks each) and the shared experts unless they
        // are dense: tiles sized for those fill the chip; the partial rows
        // stay within the workspace's max(tiles, kDenseKSplit) slots per row.
        const long long tk = (long long)T * k;
        const long long act = E < tk ? E : tk;
        const long long per = (nstar - 1 + sp.tb - 1) / sp.tb;
        const long long expect = act * per + (shared_dense ? 0 : (long long)S * ((T + sp.tb - 1) / sp.tb));
        const TilePlan tm = plan_tiles(f, (int)(expect > 0 ? expect : 1), (long long)T * (k + S), d);
        const int cap = tp.tiles > kDenseKSplit ? tp.tiles : kDenseKSplit;
        if (tm.tiles > tp.tiles && tm.tiles <= cap) tp = tm;
    }
    const int stride = mixed ? (tp.tiles > ksplit ? tp.tiles : ksplit) : 0;
    // mixed: the GEMMs go to the library stream, forked here and joined before the reduce
    std::unique_lock<std::mutex> fork_lk(g_fork_mu, std::defer_lock);
    ForkState *fs = nullptr;
    hipStream_t sg = s;
    if (mixed && use_gemm) {
        fork_lk.lock();
        fs = fork_state(s);
        if (fs) {
            if (hipEventRecord(fs->fork, s) != hipSuccess || hipStreamWaitEvent(fs->s2, fs->fork, 0) != hipSuccess)
                return MOE_ERR_HIP;
            sg = fs->s2;
        } else {
            fork_lk.unlock();
        }
    }
    if (mixed) {
        // the sparse experts: the sparse kernel over the sparse chunk table
        // (and the shared experts unless they are dense)
        SparseArgs a{};
        a.d = d; a.f = f;
        a.slots = sp.slots;
        a.cpw = tp.cpw;
        a.tiles = tp.tiles;
        a.up_q = L->up_q; a.up_sz = L->up_sz;
        a.gate = (const uint16_t *)L->gate_t; a.down = (const uint16_t *)L->down;
        a.q_stride = qs; a.sz_stride = szs; a.w_stride = wst;
        a.thr_dev = L->thresholds; a.thr = 0.f;
        a.x = (const uint16_t *)x; a.T = T;
        a.layer = 1; a.E = E; a.k = k; a.S = shared_dense ? 0 : S;
        a.chunk_tab = w.chunk_tab; a.n_chunks = w.n_chunks;
        a.offset = w.offset; a.pairs = w.pairs;
        a.topk_w = r.topk_w;
        a.part = w.part; a.part_stride = stride;
        he = launch_sparse(a, L->wdt == MOE_BF16, sp.tb, s);
        if (he != hipSuccess) return MOE_ERR_HIP;
    }
    if (use_gemm) {
        const int Sg = shared_dense ? S : 0;
        GemmArgs g{};
        g.d = d; g.f = f; g.E = E; g.k = k; g.S = Sg; g.T = T;
        g.bf16 = L->wdt == MOE_BF16 ? 1 : 0;
        g.x = (const uint16_t *)x;
        g.gate = (const uint16_t *)L->gate_t; g.up = L->up_dense;
        g.down_t = (const uint16_t *)L->down_dense;
        g.h16 = (uint16_t *)w.h; g.part = w.part; g.part_stride = stride;
        g.chunk_tab = w.chunk_tab2; g.n_chunks = w.n_chunks2; g.offset = w.offset; g.pairs = w.pairs;
        g.topk_w = r.topk_w;
        g.grid_chunks = gemm_grid_chunks(T, k, E, Sg, mt);
        g.mt = mt;
        g.ksplit = ksplit;
        he = launch_gemm_layer(g, sg);
        if (he != hipSuccess) return MOE_ERR_HIP;
        if (fs) {
            if (hipEventRecord(fs->join, sg) != hipSuccess || hipStreamWaitEvent(s, fs->join, 0) != hipSuccess)
                return MOE_ERR_HIP;
            fork_lk.unlock();
        }
        if (mixed) {
            red.tiles = tp.tiles; red.stride = stride;
            red.mix = 1; red.tiles_dense = ksplit; red.shared_dense = shared_dense ? 1 : 0;
            red.topk_idx = r.topk_idx; red.expert_dense = r.expert_dense;
        } else {
            red.tiles = ksplit;
        }
        return hip_status(launch_reduce(red, s));
    }
    if (path == MOE_PATH_DENSE) {
        DenseArgs a{};
        a.d = d; a.f = f; a.E = E; a.k = k; a.S = S; a.T = T;
        a.x = (const uint16_t *)x;
        a.gate = (const uint16_t *)L->gate_t; a.up = L->up_dense; a.down = (const uint16_t *)L->down;
        a.active = w.active; a.n_active = w.n_active; a.offset = w.offset; a.pairs = w.pairs;
        a.topk_w = r.topk_w;
        a.h = w.h; a.part = w.part;
        he = launch_dense_layer(a, s);
        if (he != hipSuccess) return MOE_ERR_HIP;
        red.tiles = kDenseKSplit;
        return hip_status(launch_reduce(red, s));
    }

    SparseArgs a{};
    a.d = d; a.f = f;
    a.slots = sp.slots;
    a.cpw = tp.cpw;
    a.tiles = tp.tiles;
    a.up_q = L->up_q; a.up_sz = L->up_sz;
    a.gate = (const uint16_t *)L->gate_t; a.down = (const uint16_t *)L->down;
    a.q_stride = qs; a.sz_stride = szs; a.w_stride = wst;
    a.thr_dev = L->thresholds; a.thr = 0.f;
    a.x = (const uint16_t *)x; a.T = T;
    a.token_scale = nullptr;
    a.layer = 1; a.E = E; a.k = k; a.S = S;
    a.chunk_tab = w.chunk_tab; a.n_chunks = w.n_chunks;
    a.chunk_rec = sp.tb == 1 ? w.chunk_rec : nullptr;
    if (inline_route) {
        a.route = 1;
        a.chunk_rec = nullptr;
        a.route_lg = inline_logits_kernel ? w.lg : nullptr;
        a.route_w = L->router_w; a.rdt = (int)L->rdt; a.route_bias = L->router_bias;
        a.renorm = L->renormalize ? 1 : 0;
        if (trace) {
            a.ex_topk_idx = trace->topk_idx; a.ex_topk_w = trace->topk_w;
            a.ex_logits = trace->logits; a.ex_count = trace->expert_count;
            a.ex_eam_row = trace->eam_row;
        }
    }
    a.offset = w.offset; a.pairs = w.pairs;
    a.topk_w = r.topk_w;
    a.part = w.part;
    const bool want_bits = trace && (trace->mask_bits || trace->nnz);
    a.mask_out = trace ? trace->masks : nullptr; a.v_out = nullptr;
    if (want_bits && !a.mask_out) a.mask_out = w.masks;
    he = launch_sparse(a, L->wdt == MOE_BF16, sp.tb, s);
    if (he != hipSuccess) return MOE_ERR_HIP;
    red.tiles = tp.tiles;
    he = launch_reduce(red, s);
    if (he == hipSuccess && want_bits)
        he = launch_mask_bits(a.mask_out, T * (k + S), f, trace->mask_bits, trace->nnz, s);
    return hip_status(he);
}

moe_status moe_pack_up_int2(const void *w_up_t, moe_dtype dt, int d, int f, uint8_t *up_q,
                            uint16_t *up_sz, void *stream)
{
    if (!w_up_t || !up_q || !up_sz) return MOE_ERR_INVALID_ARG;
    if (d < 64 || d % 64 != 0 || f < 1) return MOE_ERR_INVALID_ARG;
    if (!valid_out(dt)) return MOE_ERR_UNSUPPORTED;
    if (!aligned(up_q, 16) || !aligned(up_sz, 4) || !aligned(w_up_t, dt == MOE_F32 ? 4 : 2))
        return MOE_ERR_ALIGNMENT;
    return hip_status(launch_pack_int2(w_up_t, (int)dt, d, f, up_q, up_sz, (hipStream_t)stream));
}

moe_status moe_pack_up_bits(const void *w_up_t, moe_dtype dt, int d, int f, int bits,
                            uint8_t *up_q, uint16_t *up_sz, void *stream)
{
    if (bits == 2) return moe_pack_up_int2(w_up_t, dt, d, f, up_q, up_sz, stream);
    if (bits != 1 && bits != 4 && bits != 8) return MOE_ERR_INVALID_ARG;
    if (!w_up_t || !up_q || !up_sz) return MOE_ERR_INVALID_ARG;
    if (d < 64 || d % 64 != 0 || f < 1) return MOE_ERR_INVALID_ARG;
    if (!valid_out(dt)) return MOE_ERR_UNSUPPORTED;
    if (!aligned(up_q, 16) || !aligned(up_sz, 4) || !aligned(w_up_t, dt == MOE_F32 ? 4 : 2))
        return MOE_ERR_ALIGNMENT;
    return hip_status(launch_pack_bits(w_up_t, (int)dt, d, f, bits, up_q, up_sz,
                                       (hipStream_t)stream));
}

moe_status moe_materialize_up(const uint8_t *up_q, const uint16_t *up_sz, int d, int f,
                              moe_dtype dt, uint16_t *out, void *stream)
{
    if (!up_q || !up_sz || !out) return MOE_ERR_INVALID_ARG;
    if (d < 64 || d % 64 != 0 || f < 1) return MOE_ERR_INVALID_ARG;
    if (!is16(dt)) return MOE_ERR_UNSUPPORTED;
    if (!aligned(up_sz, 4) || !aligned(out, 2)) return MOE_ERR_ALIGNMENT;
    return hip_status(launch_materialize16(up_q, up_sz, d, f, dt == MOE_BF16, out,
                                           (hipStream_t)stream));
}

moe_status moe_materialize_up_bf16(const uint8_t *up_q, const uint16_t *up_sz, int d, int f,
                                   uint16_t *out, void *stream)
{
    return moe_materialize_up(up_q, up_sz, d, f, MOE_BF16, out, stream);
}

moe_status moe_transpose_down(const void *down, int n, int d, int f, void *out, void *stream)
{
    if (!down || !out || n < 1 || d < 1 || f < 1) return MOE_ERR_INVALID_ARG;
    if (!aligned(down, 2) || !aligned(out, 2)) return MOE_ERR_ALIGNMENT;
    return hip_status(launch_transpose16((const uint16_t *)down, n, f, d, (uint16_t *)out,
                                         (hipStream_t)stream));
}

}  // extern "C"
