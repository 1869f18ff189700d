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
// A workgroup of 8 waves (two per SIMD) computes a 256 x 256 tile; wave
// (wm, wn) owns rows 128 wm .. and 64 columns, as 4 x 2 accumulators of
// v_mfma_f32_32x32x16_{bf16,f16} (16 fp32 each), so each k step reads 4 A and
// 2 B fragments from LDS for 8 MFMAs, and one wave's MFMAs run while the
// other wave of its SIMD waits at a barrier or for LDS.  Operands move global -> LDS by DMA
// (global_load_lds_dwordx4), in blocks of 64 k values (128-byte rows) through
// two stages, one block copied while the other is multiplied; the 16-byte
// chunks of a row are XOR-swizzled so that fragment reads hit distinct banks.
// Token rows come in chunks of at most 256 (or 64, see GT) of one expert from
// the grouping kernel's chunk table.  Tiles are dealt to the XCDs so that the
// workgroups resident on one XCD share token chunks and neighbouring weight
// tiles (see the kernel).  Rows past a chunk's tokens are neither copied nor
// multiplied (their row subtiles issue no MFMAs).
#include "device.hpp"
#include "internal.hpp"

namespace moeffn {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 8;                       // 2 per SIMD: one's MFMAs cover the other's waits
constexpr int kGThreads = 64 * kWaves;
constexpr int kWNB = 16 / kWaves;               // B subtiles (32 columns) per wave
constexpr int kNT = 256;                        // tile columns (B rows)
constexpr int kKB = 64;                         // k values per stage: 128-byte rows, whole lines
constexpr int kSteps = kKB / 16;                // MFMA k steps per block
// Tile rows (tokens): MT = 256; MT = 128 with three stages (two blocks in
// flight: experts averaging up to 96 tokens, where the weight stream and its
// latency bound the kernel); MT = 64 for experts with few tokens each, whose
// 40 KB stages let two workgroups share a compute unit.
template <int MT>
struct GT {
    static constexpr int kStages = MT == 128 ? 3 : 2;
    static constexpr int kStageBytes = (MT + kNT) * kKB * 2;            // 64 / 48 / 40 KB
    static constexpr int kLds = kStages * kStageBytes;                  // 128 / 144 / 80 KB
    static constexpr int kMaxCopies = kStageBytes / 1024 / kWaves;      // copy instructions per wave
    static constexpr int kRH = MT / 2;                                  // rows per wave row-half
    static constexpr int kSub = kRH / 32;                               // row subtiles per wave
};

// s_waitcnt vmcnt(n) for a wave-uniform n in 0..7 (the copies this wave may
// leave in flight; the immediate must be a constant)
__device__ __forceinline__ void wait_vm(int n)
{
    switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    }
}

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

// Byte offset of (row, logical 16-byte chunk c) inside a stage: rows of 128
// bytes, the eight chunks XOR-swizzled by bits 0-2 of the row and bit 3, so the
// 8 (or 16) rows that a fragment read serves per LDS cycle fall in distinct
// banks (for 128- and 256-byte bank rows alike).
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int lpos(int row, int c) { return row * 128 + 16 * (c ^ swz(row)); }

struct Chunk {
    int e, ntok, pos0, hrow0;
    bool shared, valid;
};

// Chunk ci of the grid: the S shared experts' chunks of ceil(T / 256) tokens
// first, then the routed chunks listed by the grouping kernel.
template <int MT>
__device__ __forceinline__ Chunk chunk_info(const GemmArgs &a, int ci)
{
    Chunk c{};
    const int nsc = (a.T + MT - 1) / MT;
    if (ci < a.S * nsc) {
        const int sh = ci / nsc;
        const int m0 = (ci - sh * nsc) * MT;
        c.e = a.E + sh;
        c.ntok = min(MT, a.T - m0);
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
    c.ntok = min(MT, a.offset[c.e + 1] - c.pos0);
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

// The k loop of one wave over its NSUB row subtiles (those holding tokens).
// S stages: block kb + S - 1 is copied into the stage that block kb - 1 used
// while block kb is multiplied; at the end of each block the wave waits for
// its copies of block kb + 1 (leaving the later blocks' ncopy copies each in
// flight) and a barrier publishes it.  Inside a block the fragments of k step s + 1 are
// read from LDS while the MFMAs of step s run, interleaved with them
// (sched_barrier keeps the compiler from sinking the reads back next to
// their MFMAs); the other wave of each SIMD covers the rest of the waiting.
template <bool BF16, int MT, int NSUB, class ISSUE>
__device__ __forceinline__ void kloop(floatx16 (&acc)[GT<MT>::kSub][kWNB], const unsigned char *smem, int nkb,
                                      int arow0, const int (&brow)[kWNB], int li, int hk,
                                      ISSUE &issue, int ncopy)
{
    constexpr int S = GT<MT>::kStages;
    constexpr int NA = NSUB > 0 ? NSUB : 1;
    uint4 a0[NA], b0[kWNB], a1[NA], b1[kWNB];
    auto load = [&](const unsigned char *st, int step, uint4 (&af)[NA], uint4 (&bf)[kWNB]) {
        if constexpr (NSUB > 0) {
            const int c = 2 * step + hk;
#pragma unroll
            for (int j = 0; j < kWNB; ++j) bf[j] = *(const uint4 *)(st + lpos(brow[j] + li, c));
#pragma unroll
            for (int i = 0; i < NSUB; ++i) af[i] = *(const uint4 *)(st + lpos(arow0 + 32 * i + li, c));
        }
    };
    auto mmas = [&](const uint4 (&af)[NA], const uint4 (&bf)[kWNB]) {
        if constexpr (NSUB > 0) {
#pragma unroll
            for (int i = 0; i < NSUB; ++i)
#pragma unroll
                for (int j = 0; j < kWNB; ++j) acc[i][j] = mma<BF16>(af[i], bf[j], acc[i][j]);
        }
    };
    // blocks 0 .. S - 2 are issued here; block 0 must land first
#pragma unroll
    for (int b = 0; b < S - 1; ++b)
        if (b < nkb) issue(b);
    if constexpr (S == 2) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else wait_vm((nkb > S - 2 ? S - 2 : nkb - 1) * ncopy);
    __syncthreads();
    for (int kb = 0; kb < nkb; ++kb) {
        if (kb + S - 1 < nkb) issue(kb + S - 1);    // the stage block kb - 1 used
        const unsigned char *st = smem + (size_t)(kb % S) * GT<MT>::kStageBytes;
        load(st, 0, a0, b0);
        // the fragment reads of the next step are interleaved with the MFMAs
        // of this one, one read after each MFMA (sched_group_barrier: mask 8
        // MFMA, 0x100 LDS read), so that reads issue while the matrix core is busy
        constexpr int NM = (NSUB > 0 ? NSUB : 1) * kWNB, ND = (NSUB > 0 ? NSUB : 1) + kWNB;
        auto interleave = [&]() {
#pragma unroll
            for (int i = 0; i < ND; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, NM - ND > 0 ? NM - ND : 0, 0);
        };
#pragma unroll
        for (int s2 = 0; s2 < kSteps; s2 += 2) {
            load(st, s2 + 1, a1, b1);
            mmas(a0, b0);
            interleave();
            __builtin_amdgcn_sched_barrier(0);
            if (s2 + 2 < kSteps) load(st, s2 + 2, a0, b0);
            mmas(a1, b1);
            if (s2 + 2 < kSteps) interleave();
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (S == 2) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // block kb + 1 has landed
        } else {
            // blocks issued after kb + 1 may stay in flight
            const int later = (nkb - 1 < kb + S - 1 ? nkb - 1 : kb + S - 1) - (kb + 1);
            wait_vm((later > 0 ? later : 0) * ncopy);
        }
        __syncthreads();
    }
}

// MODE 0: gate/up, MODE 1: down.  MT: tile rows (256; 128 with three
// stages; 64 with two workgroups per compute unit).
template <bool BF16, int MODE, int MT>
__global__ void __launch_bounds__(kGThreads, MT == 64 ? 2 : 1)
gemm_kernel(GemmArgs a)
{
    using G = GT<MT>;
    extern __shared__ __align__(16) unsigned char smem[];
    // ---- which tile: XCD-aware.  Workgroups are dealt to the 8 XCDs in turn
    // (block b to XCD b % 8, as its (b / 8)-th).  Each XCD takes a contiguous
    // run of the tile order, whose consecutive tiles share a pair of token
    // chunks (usually one expert's) and step through neighbouring weight
    // tiles, so the workgroups resident on an XCD at one time read the same
    // token rows and each weight tile about once through that XCD's L2.
    // Tile order: chunk pair, then split-K slice, then column tile, then the
    // chunk within the pair.
    const int ntiles = MODE == 0 ? a.f / 128 : a.d / kNT;
    const int nsc = (a.T + MT - 1) / MT;
    const int vchunks = a.S * nsc + *a.n_chunks;    // chunks that hold tokens
    const int per_pair = 2 * ntiles * a.ksplit;
    const int vtiles = (vchunks + 1) / 2 * per_pair;
    const int q8 = (vtiles + 7) / 8;
    const int slot = blockIdx.x / 8;
    if (slot >= q8) return;
    const int t = (blockIdx.x % 8) * q8 + slot;
    if (t >= vtiles) return;
    const int pair = t / per_pair;
    const int r0 = t - pair * per_pair;
    const int ci = 2 * pair + (r0 & 1);
    const int nt = (r0 >> 1) % ntiles;
    const int ks = (r0 >> 1) / ntiles;              // split-K slice (down)
    if (ci >= vchunks) return;
    const Chunk ch = chunk_info<MT>(a, ci);
    if (!ch.valid) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;        // row half, column group
    const int d = a.d, f = a.f;
    const int K = MODE == 0 ? d : f;
    const int kspan = K / a.ksplit;
    const int k_beg = ks * kspan;
    const int nkb = kspan / kKB;

    // ---- copy sources.  A block is copied by 8-row instructions (1 KB of
    // the stage each): ceil(tokens / 8) for the token rows, 32 for the 256 B
    // rows; instruction q goes to wave q % kWaves, so this wave issues ncopy of
    // them per block.  Lane l of an instruction covers row base + l / 8,
    // physical chunk l % 8 (logical chunk pc ^ swizzle).  Token rows past the
    // chunk are not copied: their (stale) LDS rows only feed MFMA rows that the
    // epilogue discards.
    const int na = (min(ch.ntok, MT) + 7) / 8;
    const int ninst = na + kNT / 8;
    const int ncopy = (ninst - wave + kWaves - 1) / kWaves;
    const uint16_t *src[G::kMaxCopies];
    int dst[G::kMaxCopies];
    bool isw[G::kMaxCopies];                    // instruction copies weight rows (wave-uniform)
#pragma unroll
    for (int q = 0; q < G::kMaxCopies; ++q) {
        const int inst = min(wave + kWaves * q, ninst - 1);
        const int base = inst < na ? 8 * inst : MT + 8 * (inst - na);
        isw[q] = inst >= na;
        const int row = base + (lane >> 3);
        dst[q] = base * 128;
        const int pc = lane & 7;
        const int c = pc ^ swz(row);
        const uint16_t *rp;
        if (row < MT) {
            const int m = min(row, ch.ntok - 1);
            if (MODE == 0) rp = a.x + (size_t)token_at(a, ch, m) * d;
            else rp = a.h16 + (size_t)(ch.hrow0 + m) * f;
        } else {
            const int br = row - MT;
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
        unsigned char *base = smem + (size_t)(kb % G::kStages) * G::kStageBytes;
#pragma unroll
        for (int q = 0; q < G::kMaxCopies; ++q)
            if (q < ncopy) {
                // weight rows are streamed (nontemporal); token rows are
                // re-read by the other column tiles and stay cached
                if (isw[q]) copy16_to_lds<true>(src[q] + (size_t)kb * kKB, base + dst[q]);
                else copy16_to_lds(src[q] + (size_t)kb * kKB, base + dst[q]);
            }
    };

    floatx16 acc[G::kSub][kWNB];
#pragma unroll
    for (int i = 0; i < G::kSub; ++i)
#pragma unroll
        for (int j = 0; j < kWNB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // row subtiles of this wave that hold tokens (wave-uniform)
    const int vrows = __builtin_amdgcn_readfirstlane(ch.ntok - G::kRH * wm);
    const int nsub = vrows <= 0 ? 0 : min(G::kSub, (vrows + 31) / 32);
    // LDS rows of this wave's B subtiles
    // gate/up: the wave's gate columns first, then the same channels' up
    // columns (kWNB / 2 subtiles each); down: kWNB consecutive subtiles
    constexpr int HB = kWNB / 2;
    int brow[kWNB];
#pragma unroll
    for (int j = 0; j < kWNB; ++j) {
        if (MODE == 0) brow[j] = MT + (j < HB ? 32 * HB * wn + 32 * j : 128 + 32 * HB * wn + 32 * (j - HB));
        else brow[j] = MT + 32 * kWNB * wn + 32 * j;
    }
    const int li = lane & 31, hk = lane >> 5;

    if constexpr (G::kSub == 4) {
        switch (nsub) {
        case 4: kloop<BF16, MT, 4>(acc, smem, nkb, G::kRH * wm, brow, li, hk, issue, ncopy); break;
        case 3: kloop<BF16, MT, 3>(acc, smem, nkb, G::kRH * wm, brow, li, hk, issue, ncopy); break;
        case 2: kloop<BF16, MT, 2>(acc, smem, nkb, G::kRH * wm, brow, li, hk, issue, ncopy); break;
        case 1: kloop<BF16, MT, 1>(acc, smem, nkb, G::kRH * wm, brow, li, hk, issue, ncopy); break;
        default: kloop<BF16, MT, 0>(acc, smem, nkb, G::kRH * wm, brow, li, hk, issue, ncopy); break;
        }
    } else if constexpr (G::kSub == 2) {
        if (nsub == 2) kloop<BF16, MT, 2>(acc, smem, nkb, G::kRH * wm, brow, li, hk, issue, ncopy);
        else if (nsub == 1) kloop<BF16, MT, 1>(acc, smem, nkb, G::kRH * wm, brow, li, hk, issue, ncopy);
        else kloop<BF16, MT, 0>(acc, smem, nkb, G::kRH * wm, brow, li, hk, issue, ncopy);
    } else {
        if (nsub == 1) kloop<BF16, MT, 1>(acc, smem, nkb, G::kRH * wm, brow, li, hk, issue, ncopy);
        else kloop<BF16, MT, 0>(acc, smem, nkb, G::kRH * wm, brow, li, hk, issue, ncopy);
    }

    // ---- epilogue --------------------------------------------------------
    // value r of lane l of accumulator (i, j) is row 32 i + 8 (r / 4) + 4 hk
    // + r % 4 of the wave's rows, column 32 j + li of its columns
    if (MODE == 0) {
        if (nsub == 0) return;
#pragma unroll
        for (int i = 0; i < G::kSub; ++i) {
            if (i >= nsub) continue;
#pragma unroll
            for (int j = 0; j < HB; ++j) {
                const int col = nt * 128 + 32 * HB * wn + 32 * j + li;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = G::kRH * wm + 32 * i + 8 * (r >> 2) + 4 * hk + (r & 3);
                    if (m < ch.ntok)
                        a.h16[(size_t)(ch.hrow0 + m) * f + col] =
                            to16<BF16>(silu(acc[i][j][r]) * acc[i][j + HB][r]);
                }
            }
        }
    } else {
        // partial row and router weight of each token row of the chunk
        __syncthreads();                            // the stages are done with
        int *row_s = (int *)smem;
        float *sc_s = (float *)(smem + MT * 4);
        for (int m = tid; m < MT; m += kGThreads) {
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
        for (int i = 0; i < G::kSub; ++i) {
            if (i >= nsub) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = G::kRH * wm + 32 * i + 8 * (r >> 2) + 4 * hk + (r & 3);
                if (m >= ch.ntok) continue;
                const int pstride = a.part_stride > 0 ? a.part_stride : a.ksplit;
                float *dst = a.part + ((size_t)row_s[m] * pstride + ks) * d + (size_t)nt * kNT +
                             32 * kWNB * wn + li;
                const float sc = sc_s[m];
#pragma unroll
                for (int j = 0; j < kWNB; ++j) dst[32 * j] = sc * acc[i][j][r];
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

int gemm_grid_chunks(int T, int k, int E, int S, int mt)
{
    const long long tk = (long long)T * k;
    const long long act = E < tk ? E : tk;
    return (int)(S * ((T + mt - 1) / mt) + (tk + act * (mt - 1)) / mt);
}

namespace {
template <bool BF16, int MT>
hipError_t launch_gemm_mt(const GemmArgs &a, hipStream_t s)
{
    using G = GT<MT>;
    const void *gu = (const void *)gemm_kernel<BF16, 0, MT>;
    const void *dn = (const void *)gemm_kernel<BF16, 1, MT>;
    hipError_t e = hipFuncSetAttribute(gu, hipFuncAttributeMaxDynamicSharedMemorySize, G::kLds);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(dn, hipFuncAttributeMaxDynamicSharedMemorySize, G::kLds);
    if (e != hipSuccess) return e;
    // tiles are mapped in the kernel (XCD-aware, from the valid chunk count):
    // the grid covers the bound in pairs of chunks, 8 per XCD turn, plus 8
    const unsigned pairs = (unsigned)(a.grid_chunks + 1) / 2;
    const dim3 grid_gu((pairs * 2u * (unsigned)(a.f / 128) + 7u) / 8u * 8u + 8u);
    const dim3 grid_dn((pairs * 2u * (unsigned)(a.d / kNT) * (unsigned)a.ksplit + 7u) / 8u * 8u + 8u);
    GemmArgs gu_args = a;
    gu_args.ksplit = 1;
    hipLaunchKernelGGL((gemm_kernel<BF16, 0, MT>), grid_gu, dim3(kGThreads), G::kLds, s, gu_args);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemm_kernel<BF16, 1, MT>), grid_dn, dim3(kGThreads), G::kLds, s, a);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_layer(const GemmArgs &a, hipStream_t s)
{
    if (a.d % kNT != 0 || a.f % 128 != 0 || a.d % kKB != 0 ||
        a.f % (kKB * a.ksplit) != 0 || a.ksplit < 1 || (a.mt != 64 && a.mt != 128 && a.mt != 256))
        return hipErrorInvalidValue;
    if (a.mt == 64) return a.bf16 ? launch_gemm_mt<true, 64>(a, s) : launch_gemm_mt<false, 64>(a, s);
    if (a.mt == 128) return a.bf16 ? launch_gemm_mt<true, 128>(a, s) : launch_gemm_mt<false, 128>(a, s);
    return a.bf16 ? launch_gemm_mt<true, 256>(a, s) : launch_gemm_mt<false, 256>(a, s);
}

hipError_t launch_transpose16(const uint16_t *in, int mats, int rows, int cols, uint16_t *out,
                              hipStream_t s)
{
    const dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64), (unsigned)mats);
    hipLaunchKernelGGL(transpose16_kernel, grid, dim3(256), 0, s, in, rows, cols, out);
    return hipGetLastError();
}

}  // namespace moeffn
