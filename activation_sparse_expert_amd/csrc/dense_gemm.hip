// Dense grouped GEMM on MFMA (bf16 or fp16) for experts with many tokens
// (threshold off).  MoE-Lightning review, "层次化屋顶模型" and "MoE FFN 操作强度随
// batch/micro-batch size 增加": with many tokens per expert the expert FFN is a
// real contraction, and FloE review, "MoE 专家前向计算" gives what it computes:
//   H_e = SiLU(X_e W^gate) (.) (X_e W^up),   Y_e = H_e W^down,
// each token's row added into its output with the router weight (shared
// experts with weight 1).
//
// Both products run through one kernel shape, C = A B^T with both operands
// k-contiguous ("NT"):
//   gate/up: A = the expert's token rows of x, B = 128 gate rows followed by
//            the same 128 channels' up rows (gate_t and up_dense are stored
//            [f][d]); epilogue h = SiLU(g) u, rounded to the 16-bit type, into
//            the workspace H [pairs][f];
//   down:    A = rows of H, B = 256 rows of W^down transposed (down_dense,
//            [d][f], prepared once by moe_transpose_down); epilogue: scaled
//            by the router weight into partial rows [pair][ksplit][d], summed
//            by the reduce kernel.
// A workgroup of 4 waves computes a 256 x 256 tile; wave (wm, wn) owns rows
// 128 wm .. and 128 columns, as 4 x 4 accumulators of
// v_mfma_f32_32x32x16_{bf16,f16} (16 fp32 each), so each k step reads 4 A and
// 4 B fragments from LDS for 16 MFMAs.  Operands move global -> LDS by DMA
// (global_load_lds_dwordx4), in stages of 32 k values (64-byte rows) with
// four stages and three blocks in flight; the 16-byte chunks of a row are
// XOR-swizzled so that fragment reads hit distinct banks.  Token rows come in
// chunks of at most 256 of one expert from the grouping kernel's chunk table;
// the grid takes the chunk index fastest, so the chunks that share a weight
// tile run side by side and the tile streams from HBM about once.  Row
// subtiles past a chunk's tokens are skipped (their MFMAs are not issued);
// their rows are still copied (clamped to a valid token) to keep every wave's
// copy count fixed.
#include "device.hpp"
#include "internal.hpp"

namespace moeffn {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kGThreads = 256;                  // 4 waves
constexpr int kMT = 256;                        // tile rows (tokens)
constexpr int kNT = 256;                        // tile columns (B rows)
constexpr int kKB = 32;                         // k values per stage
constexpr int kStages = 4;
constexpr int kStageBytes = (kMT + kNT) * kKB * 2;             // 32 KB
constexpr int kGLds = kStages * kStageBytes;                    // 128 KB
constexpr int kCopies = kStageBytes / 16 / kGThreads;           // 8 per thread per stage
constexpr int kAhead = kStages - 1;

template <bool BF16>
__device__ __forceinline__ floatx16 mma(const uint4 &a, const uint4 &b, const floatx16 &c)
{
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Byte offset of (row, logical 16-byte chunk c) inside a stage: rows of 64
// bytes, the four chunks XOR-swizzled by bits 1-2 of the row, so the eight
// (or sixteen) rows a fragment read serves per LDS cycle fall in distinct banks.
__device__ __forceinline__ int lpos(int row, int c)
{
    return row * 64 + 16 * (c ^ (((row >> 1) ^ (row >> 2)) & 3));
}

struct Chunk {
    int e, ntok, pos0, hrow0;
    bool shared, valid;
};

// Chunk ci of the grid: the S shared experts' chunks of ceil(T / 256) tokens
// first, then the routed chunks listed by the grouping kernel.
__device__ __forceinline__ Chunk chunk_info(const GemmArgs &a, int ci)
{
    Chunk c{};
    const int nsc = (a.T + kMT - 1) / kMT;
    if (ci < a.S * nsc) {
        const int sh = ci / nsc;
        const int m0 = (ci - sh * nsc) * kMT;
        c.e = a.E + sh;
        c.ntok = min(kMT, a.T - m0);
        c.pos0 = m0;
        c.hrow0 = a.T * a.k + sh * a.T + m0;
        c.shared = true;
        c.valid = true;
        return c;
    }
    const int r = ci - a.S * nsc;
    c.valid = r < *a.n_chunks;
    if (!c.valid) return c;
    const int ent = a.chunk_tab[r];
    c.e = ent >> 16;
    c.pos0 = ent & 0xFFFF;
    c.ntok = min(kMT, a.offset[c.e + 1] - c.pos0);
    c.hrow0 = c.pos0;
    c.shared = false;
    return c;
}

__device__ __forceinline__ int token_at(const GemmArgs &a, const Chunk &c, int m)
{
    return c.shared ? c.pos0 + m : a.pairs[c.pos0 + m] / a.k;
}

template <bool BF16>
__device__ __forceinline__ uint16_t to16(float v)
{
    if constexpr (BF16) return float_to_bf16_bits(v);
    else return float_to_half_bits(v);
}

// The k loop of one wave over its NSUB row subtiles (those holding tokens):
// wait for block kb, publish it, refill the stage that block kb - 1 used, and
// issue the block's MFMAs from LDS fragments.
template <bool BF16, int NSUB, class ISSUE>
__device__ __forceinline__ void kloop(floatx16 (&acc)[4][4], const unsigned char *smem, int nkb,
                                      int arow0, const int (&brow)[4], int li, int hk,
                                      ISSUE &issue)
{
    for (int kb = 0; kb < nkb; ++kb) {
        // this thread's copies of block kb are done once at most the blocks
        // after it remain in flight
        const int after = min(kAhead - 1, nkb - 1 - kb);
        if (after >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kCopies) : "memory");
        else if (after == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kCopies) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        // the stage written next held block kb - 1, which every wave has finished
        if (kb + kAhead < nkb) issue(kb + kAhead);
        if constexpr (NSUB > 0) {
            const unsigned char *st = smem + (size_t)(kb % kStages) * kStageBytes;
#pragma unroll
            for (int s = 0; s < kKB / 16; ++s) {
                const int c = 2 * s + hk;
                uint4 bf[4], af[NSUB];
#pragma unroll
                for (int j = 0; j < 4; ++j) bf[j] = *(const uint4 *)(st + lpos(brow[j] + li, c));
#pragma unroll
                for (int i = 0; i < NSUB; ++i) af[i] = *(const uint4 *)(st + lpos(arow0 + 32 * i + li, c));
#pragma unroll
                for (int i = 0; i < NSUB; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = mma<BF16>(af[i], bf[j], acc[i][j]);
            }
        }
    }
}

// MODE 0: gate/up, MODE 1: down.
template <bool BF16, int MODE>
__global__ void __launch_bounds__(kGThreads)
gemm_kernel(GemmArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int nchunk_grid = a.grid_chunks;
    const int ci = blockIdx.x % nchunk_grid;
    const int rest = blockIdx.x / nchunk_grid;
    const int ntiles = MODE == 0 ? a.f / 128 : a.d / kNT;
    const int nt = rest % ntiles;
    const int ks = rest / ntiles;                   // split-K slice (down)
    const Chunk ch = chunk_info(a, ci);
    if (!ch.valid) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int d = a.d, f = a.f;
    const int K = MODE == 0 ? d : f;
    const int kspan = K / a.ksplit;
    const int k_beg = ks * kspan;
    const int nkb = kspan / kKB;

    // ---- copy sources: copy q of this thread fills stage bytes
    // (wave kCopies + q) KB + 16 lane, i.e. row (wave kCopies + q) 16 + lane / 4,
    // physical chunk lane % 4 (logical chunk pc ^ swizzle) ------------------
    const uint16_t *src[kCopies];
#pragma unroll
    for (int q = 0; q < kCopies; ++q) {
        const int row = (wave * kCopies + q) * 16 + (lane >> 2);
        const int pc = lane & 3;
        const int c = pc ^ (((row >> 1) ^ (row >> 2)) & 3);
        const uint16_t *rp;
        if (row < kMT) {
            const int m = min(row, ch.ntok - 1);        // rows past the chunk: a valid row
            if (MODE == 0) rp = a.x + (size_t)token_at(a, ch, m) * d;
            else rp = a.h16 + (size_t)(ch.hrow0 + m) * f;
        } else {
            const int br = row - kMT;
            if (MODE == 0) {
                const size_t ch0 = (size_t)ch.e * f + (size_t)nt * 128;
                rp = br < 128 ? a.gate + (ch0 + br) * d : a.up + (ch0 + br - 128) * d;
            } else {
                rp = a.down_t + ((size_t)ch.e * d + (size_t)nt * kNT + br) * f;
            }
        }
        src[q] = rp + k_beg + 8 * c;
    }
    auto issue = [&](int kb) {
        unsigned char *base = smem + (size_t)(kb % kStages) * kStageBytes;
#pragma unroll
        for (int q = 0; q < kCopies; ++q)
            copy16_to_lds(src[q] + (size_t)kb * kKB, base + (size_t)(wave * kCopies + q) * 1024);
    };

    floatx16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // row subtiles of this wave that hold tokens (wave-uniform)
    const int vrows = __builtin_amdgcn_readfirstlane(ch.ntok - 128 * wm);
    const int nsub = vrows <= 0 ? 0 : min(4, (vrows + 31) / 32);
    // LDS rows of this wave's B subtiles
    int brow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (MODE == 0) brow[j] = kMT + (j < 2 ? 64 * wn + 32 * j : 128 + 64 * wn + 32 * (j - 2));
        else brow[j] = kMT + 128 * wn + 32 * j;
    }
    const int li = lane & 31, hk = lane >> 5;

#pragma unroll
    for (int p = 0; p < kAhead; ++p)
        if (p < nkb) issue(p);
    switch (nsub) {
    case 4: kloop<BF16, 4>(acc, smem, nkb, 128 * wm, brow, li, hk, issue); break;
    case 3: kloop<BF16, 3>(acc, smem, nkb, 128 * wm, brow, li, hk, issue); break;
    case 2: kloop<BF16, 2>(acc, smem, nkb, 128 * wm, brow, li, hk, issue); break;
    case 1: kloop<BF16, 1>(acc, smem, nkb, 128 * wm, brow, li, hk, issue); break;
    default: kloop<BF16, 0>(acc, smem, nkb, 128 * wm, brow, li, hk, issue); break;
    }

    // ---- epilogue --------------------------------------------------------
    // value r of lane l of accumulator (i, j) is row 32 i + 8 (r / 4) + 4 hk
    // + r % 4 of the wave's rows, column 32 j + li of its columns
    if (MODE == 0) {
        if (nsub == 0) return;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i >= nsub) continue;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int col = nt * 128 + 64 * wn + 32 * j + li;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = 128 * wm + 32 * i + 8 * (r >> 2) + 4 * hk + (r & 3);
                    if (m < ch.ntok)
                        a.h16[(size_t)(ch.hrow0 + m) * f + col] =
                            to16<BF16>(silu(acc[i][j][r]) * acc[i][j + 2][r]);
                }
            }
        }
    } else {
        // partial row and router weight of each token row of the chunk
        __syncthreads();                            // the stages are done with
        int *row_s = (int *)smem;
        float *sc_s = (float *)(smem + kMT * 4);
        for (int m = tid; m < kMT; m += kGThreads) {
            int row = 0;
            float sc = 0.f;
            if (m < ch.ntok) {
                if (ch.shared) {
                    row = ch.hrow0 + m;
                    sc = 1.f;
                } else {
                    const int p = a.pairs[ch.pos0 + m];
                    row = p;
                    sc = a.topk_w[p];
                }
            }
            row_s[m] = row;
            sc_s[m] = sc;
        }
        __syncthreads();
        if (nsub == 0) return;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i >= nsub) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = 128 * wm + 32 * i + 8 * (r >> 2) + 4 * hk + (r & 3);
                if (m >= ch.ntok) continue;
                float *dst = a.part + ((size_t)row_s[m] * a.ksplit + ks) * d + (size_t)nt * kNT +
                             128 * wn + li;
                const float sc = sc_s[m];
#pragma unroll
                for (int j = 0; j < 4; ++j) dst[32 * j] = sc * acc[i][j][r];
            }
        }
    }
}

// out [cols][rows] = in [rows][cols] for 16-bit elements, 64 x 64 tiles
// through LDS (one-off preparation of the transposed down weights).
__global__ void __launch_bounds__(256)
transpose16_kernel(const uint16_t *in, int rows, int cols, uint16_t *out)
{
    __shared__ uint16_t t[64][66];
    const int tr = blockIdx.y * 64, tc = blockIdx.x * 64;
    const size_t mat = (size_t)blockIdx.z * rows * cols;
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        const int r = i / 64, c = i % 64;
        if (tr + r < rows && tc + c < cols) t[r][c] = in[mat + (size_t)(tr + r) * cols + tc + c];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        const int c = i / 64, r = i % 64;
        if (tr + r < rows && tc + c < cols) out[mat + (size_t)(tc + c) * rows + tr + r] = t[r][c];
    }
}

}  // namespace

int gemm_grid_chunks(int T, int k, int E, int S)
{
    const long long tk = (long long)T * k;
    const long long act = E < tk ? E : tk;
    return (int)(S * ((T + kMT - 1) / kMT) + (tk + act * (kMT - 1)) / kMT);
}

hipError_t launch_gemm_layer(const GemmArgs &a, hipStream_t s)
{
    if (a.d % kNT != 0 || a.f % 128 != 0 || a.d % kKB != 0 ||
        a.f % (kKB * a.ksplit) != 0 || a.ksplit < 1)
        return hipErrorInvalidValue;
    const void *gu = a.bf16 ? (const void *)gemm_kernel<true, 0> : (const void *)gemm_kernel<false, 0>;
    const void *dn = a.bf16 ? (const void *)gemm_kernel<true, 1> : (const void *)gemm_kernel<false, 1>;
    hipError_t e = hipFuncSetAttribute(gu, hipFuncAttributeMaxDynamicSharedMemorySize, kGLds);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(dn, hipFuncAttributeMaxDynamicSharedMemorySize, kGLds);
    if (e != hipSuccess) return e;
    GemmArgs g = a;
    const dim3 grid_gu((unsigned)a.grid_chunks * (unsigned)(a.f / 128));
    const dim3 grid_dn((unsigned)a.grid_chunks * (unsigned)(a.d / kNT) * (unsigned)a.ksplit);
    GemmArgs gu_args = g;
    gu_args.ksplit = 1;
    if (a.bf16) hipLaunchKernelGGL((gemm_kernel<true, 0>), grid_gu, dim3(kGThreads), kGLds, s, gu_args);
    else hipLaunchKernelGGL((gemm_kernel<false, 0>), grid_gu, dim3(kGThreads), kGLds, s, gu_args);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.bf16) hipLaunchKernelGGL((gemm_kernel<true, 1>), grid_dn, dim3(kGThreads), kGLds, s, g);
    else hipLaunchKernelGGL((gemm_kernel<false, 1>), grid_dn, dim3(kGThreads), kGLds, s, g);
    return hipGetLastError();
}

hipError_t launch_transpose16(const uint16_t *in, int mats, int rows, int cols, uint16_t *out,
                              hipStream_t s)
{
    const dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64), (unsigned)mats);
    hipLaunchKernelGGL(transpose16_kernel, grid, dim3(256), 0, s, in, rows, cols, out);
    return hipGetLastError();
}

}  // namespace moeffn
