// Fused activation-sparse SwiGLU expert for gfx950 (FloE review, "高效稀疏 GEMV 内核",
// Algorithm 1 and the optimisations listed after it), templated on the geometry
// of the hidden size.  Included by the per-dtype instantiation files.
//
// One workgroup owns a tile of `cpw` intermediate channels of one expert and a
// chunk of up to TB tokens, and runs the whole algorithm for them:
//   A  v = x W^up over its channels.  A lane takes 16 bytes of codes (one
//      group of 64 inputs of one channel).  fp16 activations: masking a code
//      pair in place gives an fp16 subnormal pair q 2^(p-24), so one AND per
//      pair (and one shift per word) feeds a packed dot product with fp32
//      accumulation, one accumulator per code position.  bf16 activations:
//      one mask-and-or per pair makes the bf16 pair (1 + q/4), and per group
//      sum x q = 4 (S' - X_g).  The group's share of v is s (sum x q - z X_g),
//      X_g being the group sum of x.  SEG lanes share one channel; the
//      per-channel sums of up to 8 passes are reduced together by a transposed
//      butterfly (each step halves the values a lane carries).  Code loads
//      run a few passes ahead of the decode (buffer loads over the tile;
//      passes past its end read zeros), so the VALU work overlaps the stream
//      instead of following it; with several tokens the code registers form
//      a ring that keeps the lookahead across blocks.
//   B  mask = |v| > t (fp32), union over the chunk's tokens, compacted into an
//      ascending list of active channels with a wave ballot.
//   C  for each active channel j: every thread reads its 16-byte chunk(s) of
//      gate row j and down row j (the only gate/down bytes touched), the gate
//      dot product is reduced across the workgroup, h = SiLU(g) v (fused), and
//      the thread accumulates h * down into its fp32 slice of y.
//   D  the workgroup's fp32 slice of y (scaled by the token's router weight) is
//      stored as one partial row; a second kernel sums the partials of each
//      token in a fixed order and writes the output.  No atomics, no fences:
//      the result is bit-reproducible.
// All loads are unconditional (indices clamped to valid rows, contributions of
// padding zeroed), so every load of a phase is in flight at once.
#pragma once
#include "device.hpp"
#include "internal.hpp"
#include "route_common.hpp"

namespace moeffn {
namespace sparse {

constexpr int kXPad = 72;               // halves per 64-element group slot in LDS (16 B pad)
constexpr int kPB = 8;                  // channel passes loaded and reduced together
constexpr int kAhead = 3;               // single-token tiles: passes of codes in flight
constexpr int kAheadMulti = 6;          // multi-token tiles: passes in flight (rolling)

template <int N>
struct Log2 { static constexpr int v = 1 + Log2<N / 2>::v; };
template <>
struct Log2<1> { static constexpr int v = 0; };

// Decode constants: `mask` keeps the two mantissa bits that make (1 + q/4) in
// each 16-bit half (bits 8-9 for fp16, 5-6 for bf16), `one` is the packed 1.0.
// They reach the kernel as arguments so that they sit in scalar registers: the
// compiler can then use one v_and_or_b32 per pair (gfx9 VOP3 encodings take no
// literal operands).
struct DecodeConst {
    uint32_t mask, one;
};

template <bool BF16>
__host__ __device__ constexpr DecodeConst decode_const()
{
    return BF16 ? DecodeConst{0x00600060u, 0x3F803F80u} : DecodeConst{0x03000300u, 0x3C003C00u};
}

// (a & mask) | one in one VALU instruction; mask and one are wave-uniform.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t one)
{
    uint32_t r;
    // one scalar operand at most (constant bus): `one` is kept in a vector register
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(one));
    return r;
}

// Compile-time shift that moves code slot m (bits 2m of each half-word) to the
// two mantissa bits that make (1 + q/4).
template <bool BF16, int M>
__device__ __forceinline__ uint32_t pair_word(uint32_t w, uint32_t mask, uint32_t one)
{
    constexpr int target = BF16 ? 5 : 8;
    constexpr int sh = target - 2 * M;
    uint32_t t;
    if constexpr (sh > 0) t = w << sh;
    else if constexpr (sh < 0) t = w >> (-sh);
    else t = w;
    return and_or(t, mask, one);
}

template <bool BF16>
__device__ __forceinline__ void decode_unit(const uint4 &c, uint32_t (&p)[32], uint32_t mask,
                                            uint32_t one)
{
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p[8 * i + 0] = pair_word<BF16, 0>(w[i], mask, one);
        p[8 * i + 1] = pair_word<BF16, 1>(w[i], mask, one);
        p[8 * i + 2] = pair_word<BF16, 2>(w[i], mask, one);
        p[8 * i + 3] = pair_word<BF16, 3>(w[i], mask, one);
        p[8 * i + 4] = pair_word<BF16, 4>(w[i], mask, one);
        p[8 * i + 5] = pair_word<BF16, 5>(w[i], mask, one);
        p[8 * i + 6] = pair_word<BF16, 6>(w[i], mask, one);
        p[8 * i + 7] = pair_word<BF16, 7>(w[i], mask, one);
    }
}

// sum_k x_k (1 + q_k/4) over one 64-input group: 32 packed dot products in four
// independent chains
template <bool BF16>
__device__ __forceinline__ float group_dot(const uint32_t (&pw)[32], const uint32_t (&xp)[32])
{
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int m = 0; m < 32; m += 4) {
        a0 = dot2<BF16>(pw[m], xp[m], a0);
        a1 = dot2<BF16>(pw[m + 1], xp[m + 1], a1);
        a2 = dot2<BF16>(pw[m + 2], xp[m + 2], a2);
        a3 = dot2<BF16>(pw[m + 3], xp[m + 3], a3);
    }
    return (a0 + a1) + (a2 + a3);
}

// sum_k x_k q_k over one 64-input group, fp16 activations.  Masking a code
// pair in place leaves an fp16 subnormal pair q 2^(p-24) (p = bit position of
// the code in its half-word, 0..8): one v_and_b32 per pair for code slots 0-4,
// and one shift of the word by 6 brings slots 5-7 to positions 4, 6, 8.  Pairs
// with the same position share an accumulator, and the positions are
// recombined by exact powers of two.  Measured on gfx950 with activations of
// the N(0,1)/64 scale: the packed dot product keeps a relative error of about
// 1e-6 on the position-0 chain and 1e-8 on positions 4-8 (the latter carry
// 16-256x the weight), and it does not flush fp16 subnormal inputs; there is
// no cancellation against a constant term as in the (1 + q/4) decode.
__device__ __forceinline__ float group_xq_f16(const uint4 &c, const uint32_t (&xp)[32])
{
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    float a0 = 0.f, a2 = 0.f, a4 = 0.f, a6 = 0.f, a8 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t wi = w[i], ws = wi >> 6;
        a0 = dot2<false>(wi & 0x00030003u, xp[8 * i + 0], a0);
        a2 = dot2<false>(wi & 0x000C000Cu, xp[8 * i + 1], a2);
        a4 = dot2<false>(wi & 0x00300030u, xp[8 * i + 2], a4);
        a6 = dot2<false>(wi & 0x00C000C0u, xp[8 * i + 3], a6);
        a8 = dot2<false>(wi & 0x03000300u, xp[8 * i + 4], a8);
        a4 = dot2<false>(ws & 0x00300030u, xp[8 * i + 5], a4);
        a6 = dot2<false>(ws & 0x00C000C0u, xp[8 * i + 6], a6);
        a8 = dot2<false>(ws & 0x03000300u, xp[8 * i + 7], a8);
    }
    return 65536.0f * ((((a0 * 4.0f + a2) * 4.0f + a4) * 4.0f + a6) * 4.0f + a8);
}

// The activation pairs of one group: from registers (XREG) or from the copy
// just read out of LDS.
template <bool XREG, int N>
__device__ __forceinline__ const uint32_t (&pick_x(const uint32_t (&reg)[32],
                                                   const uint32_t (&lds)[N]))[32]
{
    if constexpr (XREG) return reg;
    else return lds;
}

// Transposed butterfly over the SEG lanes of a segment: on entry every lane
// holds P partial values (P a power of two <= SEG); on exit value 0 of a lane is
// the segment total of value index (go >> (log2 SEG - log2 P)), go being the
// lane's position in the segment.  Each step at stride S halves the values a
// lane carries (it keeps one half and receives its partner's copy of that
// half); once one value is left the remaining strides are plain butterflies.
// Fixed order: bit-reproducible.
template <int P, int S, int N>
__device__ __forceinline__ float treduce_step(float (&v)[P], int lane)
{
    if constexpr (S == 0) {
        return v[0];
    } else if constexpr (S >= 16) {
        if constexpr (N > 1) {
#pragma unroll
            for (int i = 0; i < N / 2; ++i) v[i] = swap_add<S>(v[i], v[i + N / 2]);
            return treduce_step<P, S / 2, N / 2>(v, lane);
        } else {
            v[0] = swap_add<S>(v[0], v[0]);
            return treduce_step<P, S / 2, 1>(v, lane);
        }
    } else {
        const bool hi = (lane & S) != 0;
        if constexpr (N > 1) {
#pragma unroll
            for (int i = 0; i < N / 2; ++i) {
                const float send = hi ? v[i] : v[i + N / 2];
                const float keep = hi ? v[i + N / 2] : v[i];
                v[i] = keep + xor_lane<S>(send);
            }
            return treduce_step<P, S / 2, N / 2>(v, lane);
        } else {
            v[0] += xor_lane<S>(v[0]);
            return treduce_step<P, S / 2, 1>(v, lane);
        }
    }
}

template <int P, int SEG>
__device__ __forceinline__ float transposed_reduce(float (&v)[P], int lane)
{
    static_assert(P <= SEG || SEG == 1, "values per lane exceed the segment");
    return treduce_step<P, SEG / 2, P>(v, lane);
}

struct Lds {
    uint16_t *xs;       // [TB][G][kXPad] activations (16-bit), group-padded
    float *xg;          // [TB][G] group sums of x
    float *vs;          // [TB][cpw]
    uint8_t *mk;        // [TB][cpw]
    uint16_t *list;     // [cpw] active channels (union over the chunk's tokens)
    float *gp;          // [W][RB][TB] partial gate dots
    int32_t *tok_t;     // [TB] token index
    int32_t *tok_slot;  // [TB] mask slot (layer mode)
    int32_t *tok_row;   // [TB] partial row
    float *tok_sc;      // [TB] scale
    int32_t *misc;      // [0] n_act
    float *rlg;         // [E rounded up to 4] logits (inline routing)
    int32_t *rsel;      // [k] the token's choices (inline routing)
};

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// LDS bytes of the inline routing: E logits (padded to 4) and k choices
__host__ __device__ inline size_t route_lds(int E, int k) { return (size_t)(((E + 3) & ~3) + k) * 4; }

__host__ __device__ inline size_t lds_layout(int d, int cpw, int tb, int waves, int rb, size_t *off,
                                             size_t route_bytes = 0)
{
    const int G = d / 64;
    size_t o = 0;
    off[0] = o; o = align16(o + (size_t)tb * G * kXPad * 2);
    off[1] = o; o = align16(o + (size_t)tb * G * 4);
    off[2] = o; o = align16(o + (size_t)tb * cpw * 4);
    off[3] = o; o = align16(o + (size_t)tb * cpw);
    off[4] = o; o = align16(o + (size_t)cpw * 2);
    off[5] = o; o = align16(o + (size_t)waves * rb * tb * 4);
    off[6] = o; o = align16(o + (size_t)tb * 4);
    off[7] = o; o = align16(o + (size_t)tb * 4);
    off[8] = o; o = align16(o + (size_t)tb * 4);
    off[9] = o; o = align16(o + (size_t)tb * 4);
    off[10] = o; o = align16(o + 16);
    off[11] = o; o = align16(o + route_bytes);
    return o;
}

// Compile-time geometry for a hidden size class.
//   SEG     lanes sharing one channel in phase A (the power of two >= d/64
//           when d <= 4096; lanes past d/64 groups read zeros)
//   NG      64-input groups per lane in phase A
//   NCH     16-byte column chunks per thread in phase C
//   THREADS workgroup size
template <int SEG_, int NG_, int NCH_, int THREADS_>
struct Geo {
    static constexpr int SEG = SEG_, NG = NG_, NCH = NCH_, THREADS = THREADS_;
    static constexpr int W = THREADS / 64;
};

// Gate/down rows gathered per batch in phase C.  Each batch costs at least one
// memory round trip and the workgroup with the most active rows sets the
// kernel's duration, so a single token takes 16 rows at once (about three
// standard deviations above the mean at 90% sparsity and 56 channels).
template <int TB, int NCH>
__host__ __device__ constexpr int rows_per_batch()
{
    if (TB == 1 && NCH == 1) return 16;
    return (8 / NCH) < 1 ? 1 : 8 / NCH;
}

// Raw buffer access to one tile's codes or scales: offsets at or past
// `bytes` (kOob) return zeros without a memory access, so the loads of a
// block of passes can be issued unconditionally.
constexpr uint32_t kOob = 0x7FFFFFF0u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ uint4 bload_nt16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2 /* nt */);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t bload_nt4(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 2 /* nt */);
}

// ---- other up-code widths (FloE review, "敏感度分析": INT8, INT4, INT1) ----
// The codes are packed plainly: input k of a channel at bits [k b, k b + b) of
// its row, with the same group-64 scale and zero point as the INT2 format.  A
// lane still takes one 64-input group (2 b code words).  In a code word the
// two 16-bit halves hold inputs at the same bit position, so a mask and a
// shift that put those two codes at the top of an fp16 mantissa give an
// fp16 subnormal pair q 2^(top - 24) (bf16: a normal pair 1 + q 2^-n),
// which one packed dot product multiplies with the matching pair of x.  The
// lane's x pairs are permuted once to that order (perm_pairs).
template <int BITS>
struct CodeUnit {
    uint32_t w[2 * BITS];
};
template <>
struct CodeUnit<2> {
    uint4 v;
};

template <int BITS>
__device__ __forceinline__ CodeUnit<BITS> bload_codes(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    CodeUnit<BITS> c;
    if constexpr (BITS == 2) {
        c.v = bload_nt16(r, off);
    } else if constexpr (BITS == 1) {
        typedef uint32_t v2u __attribute__((ext_vector_type(2)));
        const v2u v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 2 /* nt */);
        c.w[0] = v.x;
        c.w[1] = v.y;
    } else {
#pragma unroll
        for (int i = 0; i < BITS / 2; ++i) {
            // an offset past the tile stays past it: every part reads zeros
            const uint4 u = bload_nt16(r, off >= kOob ? kOob : off + 16u * i);
            c.w[4 * i] = u.x;
            c.w[4 * i + 1] = u.y;
            c.w[4 * i + 2] = u.z;
            c.w[4 * i + 3] = u.w;
        }
    }
    return c;
}

// x pairs in the order the BITS-wide code words pair their inputs, from the
// natural pairs n[j] = (x[2j], x[2j+1]) of one 64-input group.  Word i of the
// codes covers inputs 32 i / b ...; its pair m holds inputs (i0 + m, i0 + m +
// 16 / b) (lo, hi half).  v_perm_b32 takes 16-bit halves of two natural pairs.
template <int BITS>
__device__ __forceinline__ void perm_pairs(uint32_t (&xp)[32])
{
    if constexpr (BITS != 2) {
        uint32_t n[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) n[j] = xp[j];
        constexpr int IW = 32 / BITS;               // inputs per code word
        constexpr int H = IW / 2;                   // inputs per half word (pairs per word)
#pragma unroll
        for (int i = 0; i < 2 * BITS; ++i)
#pragma unroll
            for (int m = 0; m < H; ++m) {
                const int lo = i * IW + m, hi = lo + H;          // inputs of pair (i, m)
                // both have the parity of m: the low half of their natural pair if even
                const uint32_t sel = (m & 1) ? 0x07060302u : 0x05040100u;
                xp[i * H + m] = __builtin_amdgcn_perm(n[hi >> 1], n[lo >> 1], sel);
            }
    }
}

// sum_k x_k q_k over one group for BITS in {8, 4, 1}, fp16 activations: each
// pair of codes moved to mantissa bits [10 - b', 10) (b' = min(b, 8)) as a
// subnormal pair, four accumulators, one exact power of two at the end.
template <int BITS>
__device__ __forceinline__ float group_xq_bits_f16(const CodeUnit<BITS> &c, const uint32_t (&xp)[32])
{
    if constexpr (BITS == 1) {
        // one bit per code: bit m of each half is the subnormal 2^(m - 24) as
        // it stands (m <= 9); bits 10..15 are shifted down by 6, to positions
        // 4..9.  One accumulator per position, exact powers of two at the end.
        float acc[10];
#pragma unroll
        for (int p = 0; p < 10; ++p) acc[p] = 0.f;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t w = c.w[i], ws = w >> 6;
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const int p = m < 10 ? m : m - 6;
                const uint32_t pw = (m < 10 ? w : ws) & (0x00010001u << p);
                acc[p] = dot2<false>(pw, xp[i * 16 + m], acc[p]);
            }
        }
        float r = 0.f;
#pragma unroll
        for (int p = 0; p < 10; ++p) r += acc[p] * (float)(1u << (24 - p));
        return r;
    }
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    constexpr int H = 16 / BITS;                    // pairs per code word
#pragma unroll
    for (int i = 0; i < 2 * BITS; ++i) {
        const uint32_t w = c.w[i];
#pragma unroll
        for (int m = 0; m < H; ++m) {
            constexpr int top = 10;                 // codes end at mantissa bit 9
            const int sh = top - BITS * (m + 1);    // shift that moves pair m there
            const uint32_t mask = ((1u << BITS) - 1u) << (top - BITS);
            const uint32_t t = sh >= 0 ? (w << sh) : (w >> (-sh));
            const uint32_t pw = t & (mask | (mask << 16));
            acc[(i * H + m) & 3] = dot2<false>(pw, xp[i * H + m], acc[(i * H + m) & 3]);
        }
    }
    // a code q sits at q 2^(top - b - 24) = q 2^-(14 + b)
    return ((acc[0] + acc[1]) + (acc[2] + acc[3])) * (float)(1u << (14 + BITS));
}

// bf16 activations: pair words (1 + q 2^-n) from one v_and_or per pair, the
// code placed at mantissa bits [7 - b', 7); sum x q = 2^n (S' - X_g).  Eight
// bits are taken as two nibbles, 16 (S'_lo - X_g) + 256 (S'_hi - X_g).
template <int BITS>
__device__ __forceinline__ float group_xq_bits_bf16(const CodeUnit<BITS> &c, const uint32_t (&xp)[32],
                                                    float xg, uint32_t one)
{
    constexpr int NB = BITS == 8 ? 4 : BITS;        // bits per decoded field
    constexpr int NF = BITS == 8 ? 2 : 1;           // fields per code
    constexpr int H = 16 / BITS;
    constexpr uint32_t fmask = ((1u << NB) - 1u) << (7 - NB);
    float acc[NF][2];
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[f][0] = acc[f][1] = 0.f;
#pragma unroll
    for (int i = 0; i < 2 * BITS; ++i) {
        const uint32_t w = c.w[i];
#pragma unroll
        for (int m = 0; m < H; ++m)
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const int sh = 7 - (BITS * m + NB * f + NB);  // field's top bit to mantissa bit 6
                const uint32_t t = sh >= 0 ? (w << sh) : (w >> (-sh));
                const uint32_t pw = and_or(t, fmask | (fmask << 16), one);
                acc[f][m & 1] = dot2<true>(pw, xp[i * H + m], acc[f][m & 1]);
            }
    }
    // field f (value v) reads 1 + v 2^-NB and weighs 2^(NB f) in the code
    float r = 0.f;
#pragma unroll
    for (int f = 0; f < NF; ++f) r += ((acc[f][0] + acc[f][1]) - xg) * (float)(1u << (NB * (f + 1)));
    return r;
}

// Gate/down row chunk of phase C.  A single-token chunk reads each active row
// once, so the rows are streamed (nontemporal); chunks of several tokens keep
// ordinary loads, because other chunks of the same expert read the same rows
// and find them in cache (and load from a buffer over the tile's rows, where
// an offset of kOob reads zeros without a memory access).
__device__ __forceinline__ uint4 row_load_nt(const uint16_t *p) { return load_nt16(p); }
__device__ __forceinline__ uint4 row_bload(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// passes of channels per phase-A block (host and device).  A single-token
// block holds kPB / NG passes.  A multi-token block holds the same number of
// passes as a ring of code registers: the loads run kAheadMulti passes
// ahead across block boundaries, so each lane keeps that many 16-byte units
// in flight however many tokens the chunk holds.
// Other code widths hold 2 BITS code words per group: a block holds at most
// 32 code words per lane and kPB passes (2 passes at 8 bits, 4 at 4 bits).
template <int TB, class GEO, int BITS = 2>
__host__ __device__ constexpr int pass_block()
{
    constexpr int per = 2 * BITS * GEO::NG;                 // code words per pass and lane
    constexpr int pw = (32 / per) < 1 ? 1 : (32 / per);
    constexpr int pb = BITS == 2 ? ((kPB / GEO::NG) < 1 ? 1 : (kPB / GEO::NG))
                                 : (pw < kPB ? pw : kPB);
    return pb < GEO::SEG ? pb : GEO::SEG;
}

// Inline routing of a single token (layer calls at T = 1): the logits come
// from the logits kernel or are formed here, one wave per expert; then the
// shared ranking and gate weights, exactly as the routing kernel forms them.
// Returns this slot's expert and weight; the writer workgroup also writes the
// trace exports (choices, weights, logits, per-expert counts, EAM row).
template <bool BF16, int THREADS>
__device__ __forceinline__ void route_token(const SparseArgs &a, const Lds &L, int slot, bool writer,
                                            int tid, int lane, int wave, int &e, float &w)
{
    constexpr int W = THREADS / 64;
    const int E = a.E, k = a.k, E4 = (E + 3) & ~3;
    float *lg = L.rlg;
    int32_t *sel = L.rsel;
    if (a.route_lg) {
        for (int i = tid; i < E; i += THREADS) lg[i] = a.route_lg[i];
    } else {
        for (int i = wave; i < E; i += W) {
            const float v = rc::wave_logit_rows<BF16 ? 1 : 0>(a.x, a.route_w, a.rdt, a.d,
                                                              a.route_bias, i, lane);
            if (lane == 0) lg[i] = v;
        }
    }
    for (int i = E + tid; i < E4; i += THREADS) lg[i] = -INFINITY;
    __syncthreads();
    rc::rank_topk(lg, E, k, sel, tid, THREADS);
    __syncthreads();
    const float m = lg[sel[0]];
    const float den = rc::gate_den(lg, sel, E, k, a.renorm, m, lane);
    e = sel[slot];
    w = __expf(lg[e] - m) / den;
    if (writer) {
        for (int s = tid; s < k; s += THREADS) {
            if (a.ex_topk_idx) a.ex_topk_idx[s] = sel[s];
            if (a.ex_topk_w) a.ex_topk_w[s] = __expf(lg[sel[s]] - m) / den;
        }
        for (int i = tid; i < E; i += THREADS) {
            if (a.ex_logits) a.ex_logits[i] = lg[i];
            int c = 0;
            for (int s = 0; s < k; ++s) c |= (int)(sel[s] == i);
            if (a.ex_count) a.ex_count[i] = c;
            if (a.ex_eam_row && c) a.ex_eam_row[i] += 1;
        }
    }
}

// ONE: the tile is a single block of passes (straight-line code).  PBX: the
// block is PBX times the usual pass block (2 for single-token tiles of 9-16
// passes, so that they too run straight-line with a continuous lookahead).
template <bool BF16, int TB, class GEO, bool ONE, int PBX = 1, bool ROUTE = false, int BITS = 2>
__global__ void __launch_bounds__(GEO::THREADS)
expert_kernel(SparseArgs a)
{
    constexpr int SEG = GEO::SEG, NG = GEO::NG, NCH = GEO::NCH, THREADS = GEO::THREADS;
    constexpr int W = GEO::W;
    constexpr int RPW = 64 / SEG;                   // channels per wave pass
    constexpr int ROWS_PASS = W * RPW;              // channels per workgroup pass
    constexpr int RB = rows_per_batch<TB, NCH>();
    constexpr int LOGSEG = Log2<SEG>::v;
    // channel passes loaded and reduced together (<= SEG; fewer when a lane
    // carries several tokens or groups, to bound registers)
    constexpr int PR = pass_block<TB, GEO, BITS>() * PBX;
    static_assert(PR <= GEO::SEG, "passes of a block exceed the segment");
    constexpr bool XREG = (TB * NG) <= 4;            // x pairs of the lane's groups kept in registers
    static_assert(BITS == 2 || XREG, "other code widths keep x in registers");
    constexpr int QB = 8 * BITS;                     // code bytes per 64-input group

    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int d = a.d, f = a.f, G = d / 64;
    const int cpw = a.cpw;

    size_t off[12];
    lds_layout(d, cpw, TB, W, RB, off, ROUTE ? route_lds(a.E, a.k) : 0);
    Lds L;
    L.xs = (uint16_t *)(smem + off[0]);
    L.xg = (float *)(smem + off[1]);
    L.vs = (float *)(smem + off[2]);
    L.mk = (uint8_t *)(smem + off[3]);
    L.list = (uint16_t *)(smem + off[4]);
    L.gp = (float *)(smem + off[5]);
    L.tok_t = (int32_t *)(smem + off[6]);
    L.tok_slot = (int32_t *)(smem + off[7]);
    L.tok_row = (int32_t *)(smem + off[8]);
    L.tok_sc = (float *)(smem + off[9]);
    L.misc = (int32_t *)(smem + off[10]);
    L.rlg = (float *)(smem + off[11]);
    L.rsel = (int32_t *)(L.rlg + ((a.E + 3) & ~3));

    // ---- which expert and which tokens ------------------------------------
    // The grid is (token chunk) x (tile).  Single expert: chunk c holds tokens
    // c TB ..; layer: the S shared experts' chunks of every token come first,
    // then the routed chunks listed by the grouping kernel.
    const int chunk = blockIdx.x / a.tiles;
    const int tile = blockIdx.x - chunk * a.tiles;
    int e = 0, nt = 0, pos0 = 0, tbase = 0, sh = 0;
    int rec_p = -1;                                 // single-token chunk record: pair, weight
    float rec_w = 1.0f;
    bool shared_slot = false;
    if (!a.layer) {
        tbase = chunk * TB;
        nt = min(TB, a.T - tbase);
    } else {
        const int nsc = (a.T + TB - 1) / TB;        // chunks per shared expert
        if (chunk < a.S * nsc) {
            sh = chunk / nsc;
            tbase = (chunk - sh * nsc) * TB;
            nt = min(TB, a.T - tbase);
            e = a.E + sh;
            shared_slot = true;
        } else {
            const int ci = chunk - a.S * nsc;
            if constexpr (ROUTE) {
                // one token, slot ci: rank its logits here
                route_token<BF16, THREADS>(a, L, ci, ci == 0 && tile == 0, tid, lane, wave, e, rec_w);
                rec_p = ci;                         // pair ci of token 0
                nt = 1;
            } else if (TB == 1 && a.chunk_rec) {
                // one pair per chunk: the grid holds exactly T k routed chunks
                const int4 rec = *(const int4 *)(a.chunk_rec + 4 * (size_t)ci);
                e = rec.x;
                rec_p = rec.y;
                rec_w = __int_as_float(rec.z);
                pos0 = rec.w;
                nt = 1;
            } else {
                if (ci >= *a.n_chunks) return;      // beyond this call's chunks
                const int ent = a.chunk_tab[ci];
                e = ent >> 16;
                pos0 = ent & 0xFFFF;
                nt = min(TB, a.offset[e + 1] - pos0);
            }
        }
    }
    if (nt <= 0) return;
    const float thr = a.thr_dev ? a.thr_dev[e] : a.thr;
    const int j0 = tile * cpw;
    const int nrows = min(cpw, f - j0);
    if (nrows <= 0) return;

    const int rowb = d * BITS / 8;                   // code bytes per channel
    const uint8_t *upq = a.up_q + (size_t)e * a.q_stride + (size_t)j0 * rowb;
    const uint16_t *upsz = a.up_sz + (size_t)e * a.sz_stride + (size_t)j0 * G * 2;
    const uint16_t *gate = a.gate + (size_t)e * a.w_stride + (size_t)j0 * d;
    const uint16_t *down = a.down + (size_t)e * a.w_stride + (size_t)j0 * d;

    const int go = lane & (SEG - 1);                // position in the channel's segment
    const int rs = lane / SEG;                      // segment (channel slot) in the wave
    const int passes = (nrows + ROWS_PASS - 1) / ROWS_PASS;
    const int CPR = d / 8;                          // 16-byte chunks per d-row

    // phase-A code units of one block of PR passes (slot p holds pass p0 + p)
    CodeUnit<BITS> cq[PR][NG];
    uint32_t csz[PR][NG];
    // The loads run AH passes ahead of the decode, as raw buffer loads over
    // the tile (passes past its end read zeros without a memory access), so no
    // branch separates them and the compiler's wait counts stay exact.  Single
    // token: the passes of a block are issued AH at a time from its start.
    // Several tokens (RING): the pass AH ahead goes into the slot freed by the
    // pass just decoded, across block boundaries, so the stream never drains.
    constexpr bool RING = TB > 1 || BITS != 2;
    constexpr int AH = RING ? (kAheadMulti < PR ? kAheadMulti : PR - 1)
                            : (kAhead < PR ? kAhead : PR);
    static_assert(AH >= 1 || PR == 1, "lookahead");
    constexpr int PRED = (TB >= 4 && PR >= 2) ? PR / 2 : PR;
    const __amdgpu_buffer_rsrc_t rq = tile_rsrc(upq, (uint32_t)nrows * rowb);
    const __amdgpu_buffer_rsrc_t rz = tile_rsrc(upsz, (uint32_t)nrows * G * 4);
    const int r_lane = wave * RPW + rs;             // channel of this lane in pass 0
    const uint32_t q_lane = (uint32_t)(r_lane * rowb + go * QB);
    const uint32_t z_lane = (uint32_t)((r_lane * G + go) * 4);
#define LOAD_SLOT(PP, SLOT)                                                                 \
    {                                                                                       \
        const int pp = (PP);                                                                \
        const bool rok = r_lane + pp * ROWS_PASS < nrows;                                   \
        _Pragma("unroll") for (int gi = 0; gi < NG; ++gi) {                                 \
            const bool ok = rok && go + SEG * gi < G;                                       \
            const uint32_t oq = q_lane + (uint32_t)(pp * ROWS_PASS * rowb + gi * SEG * QB);  \
            const uint32_t oz = z_lane + (uint32_t)((pp * ROWS_PASS * G + gi * SEG) * 4);   \
            cq[SLOT][gi] = bload_codes<BITS>(rq, ok ? oq : kOob);                           \
            csz[SLOT][gi] = bload_nt4(rz, ok ? oz : kOob);                                  \
        }                                                                                   \
    }
#define LOAD_PASS(P0, p) LOAD_SLOT((P0) + (p), p)

    // 16-byte x chunks each thread stages per token chunk
    constexpr int XL = (TB * 8 * SEG * NG + THREADS - 1) / THREADS;

    // ---- token bookkeeping (small loads, before the streams start) --------
    if (tid < TB) {
        int t = 0, sl = 0, row = 0;
        float sc = 1.0f;                            // router weight / caller's scale
        if (tid < nt) {
            if (!a.layer) {
                t = tbase + tid;
                row = t;
                if (a.token_scale) sc = a.token_scale[t];
            } else if (shared_slot) {
                t = tbase + tid;
                sl = a.k + sh;
                row = a.T * a.k + sh * a.T + t;
            } else {
                const int pos = pos0 + tid;
                const int p = rec_p >= 0 ? rec_p : a.pairs[pos];
                t = p / a.k;
                sl = p - t * a.k;
                row = p;                            // routed partial rows are indexed by pair
                sc = rec_p >= 0 ? rec_w : a.topk_w[p];
            }
        }
        L.tok_t[tid] = t;
        L.tok_slot[tid] = sl;
        L.tok_row[tid] = row;
        L.tok_sc[tid] = sc;
    }
    // a single token known without the table (single expert, shared expert,
    // chunk record): its x load need not wait for the bookkeeping (the
    // x-staging barrier publishes it before any use)
    const int t0u = TB > 1 ? -1
                  : (!a.layer || shared_slot) ? tbase : (rec_p >= 0 ? rec_p / a.k : -1);
    if (t0u < 0) __syncthreads();

    // ---- x loads, then the up-code loads; only x is waited for here -------
    uint4 xl[XL];
    if constexpr (TB == 1) {
        // one token: a buffer over its row, so that no branch separates the
        // x load from the code loads issued after it
        const int t0 = t0u >= 0 ? t0u : __builtin_amdgcn_readfirstlane(L.tok_t[0]);
        const __amdgpu_buffer_rsrc_t rx = tile_rsrc(a.x + (size_t)t0 * d, (uint32_t)d * 2);
#pragma unroll
        for (int u = 0; u < XL; ++u) {
            const int i = tid + u * THREADS;
            typedef uint32_t v4u __attribute__((ext_vector_type(4)));
            const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rx, i < CPR ? i * 16 : (int)kOob, 0, 0);
            xl[u] = make_uint4(v.x, v.y, v.z, v.w);
        }
    } else {
#pragma unroll
        for (int u = 0; u < XL; ++u) {
            const int i = tid + u * THREADS;
            const int tb = i / CPR, c = i - tb * CPR;
            xl[u] = make_uint4(0, 0, 0, 0);
            if (i < TB * CPR && tb < nt) xl[u] = *(const uint4 *)(a.x + (size_t)L.tok_t[tb] * d + (size_t)c * 8);
        }
    }
    // up codes do not depend on x: in flight while x is staged (x first)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 0; p < AH; ++p) {
        LOAD_PASS(0, p)
        __builtin_amdgcn_sched_barrier(0);          // keep the passes in order
    }
#pragma unroll
    for (int u = 0; u < XL; ++u) {
        const int i = tid + u * THREADS;
        const int tb = i / CPR, c = i - tb * CPR;
        if (i < TB * CPR)
            *(uint4 *)(L.xs + ((size_t)tb * G + (c >> 3)) * kXPad + (c & 7) * 8) = xl[u];
    }
    __syncthreads();
    if constexpr (!XREG) {
        for (int i = tid; i < TB * G; i += THREADS) {
            const uint32_t *xp = (const uint32_t *)(L.xs + (size_t)i * kXPad);
            float s0 = 0.f, s1 = 0.f;
#pragma unroll 8
            for (int m = 0; m < 32; ++m) {
                s0 += lo16_to_float<BF16>(xp[m]);
                s1 += hi16_to_float<BF16>(xp[m]);
            }
            L.xg[i] = s0 + s1;
        }
        __syncthreads();
    }

    // ---- A: v = x W^up for this tile ------------------------------------
    // With the lane's x pairs in registers (XREG) the group sums come from
    // them (packed dot with ones, no further barrier); otherwise from LDS.
    uint32_t xr_a[XREG ? TB * NG : 1][32];
    float xg_a[TB][NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        const int g = min(go + SEG * gi, G - 1);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            if constexpr (XREG) {
                const uint4 *xv = (const uint4 *)(L.xs + ((size_t)tb * G + g) * kXPad);
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const uint4 xx = xv[q];
                    xr_a[tb * NG + gi][4 * q + 0] = xx.x;
                    xr_a[tb * NG + gi][4 * q + 1] = xx.y;
                    xr_a[tb * NG + gi][4 * q + 2] = xx.z;
                    xr_a[tb * NG + gi][4 * q + 3] = xx.w;
                }
                float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
                for (int m = 0; m < 32; m += 4) {
                    s0 = dot2<BF16>(xr_a[tb * NG + gi][m], a.dec_one, s0);
                    s1 = dot2<BF16>(xr_a[tb * NG + gi][m + 1], a.dec_one, s1);
                    s2 = dot2<BF16>(xr_a[tb * NG + gi][m + 2], a.dec_one, s2);
                    s3 = dot2<BF16>(xr_a[tb * NG + gi][m + 3], a.dec_one, s3);
                }
                xg_a[tb][gi] = (s0 + s1) + (s2 + s3);
                perm_pairs<BITS>(xr_a[tb * NG + gi]);   // the code words' pair order
            } else {
                xg_a[tb][gi] = L.xg[tb * G + g];
            }
        }
    }
    // ONE: the tile is a single block of passes (straight-line code)
    for (int p0 = 0; p0 < (ONE ? 1 : passes); p0 += PR) {
        if constexpr (!RING && !ONE) {
            if (p0 > 0) {
#pragma unroll
                for (int p = 0; p < AH; ++p) LOAD_PASS(p0, p)
            }
        }
        // The passes' per-lane sums are reduced over the segment's lanes in
        // groups of PRED passes (half a block with four tokens, to bound
        // registers), right after the group's last pass.
        float part[TB][PRED];
#pragma unroll
        for (int p = 0; p < PR; ++p) {
            const int pg = p % PRED;
            if (pg == 0) {
#pragma unroll
                for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                    for (int q = 0; q < PRED; ++q) part[tb][q] = 0.f;
            }
            if constexpr (RING) {
                // slot (p + AH) % PR was decoded at pass p + AH - PR of this block
                if (!ONE || p + AH < PR) LOAD_SLOT(p0 + p + AH, (p + AH) % PR)
            } else {
                if (p + AH < PR) LOAD_PASS(p0, p + AH)
            }
            __builtin_amdgcn_sched_barrier(0);
            if (p0 + p < passes) {                  // uniform: padding passes of the block
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    // fp16: subnormal-pair decode (group_xq_f16); bf16: (1 + q/4) pairs
                    uint32_t pw[BF16 && BITS == 2 ? 32 : 1];
                    if constexpr (BF16 && BITS == 2) decode_unit<BF16>(cq[p][gi].v, pw, a.dec_mask, a.dec_one);
                    // units outside the tile read zeros from the buffer loads: s = 0
                    const float s = half_bits_to_float(csz[p][gi] & 0xFFFFu);
                    const float z = half_bits_to_float(csz[p][gi] >> 16);
                    const int g = min(go + SEG * gi, G - 1);
#pragma unroll
                    for (int tb = 0; tb < TB; ++tb) {
                        uint32_t xl_[XREG ? 1 : 32];
                        if constexpr (!XREG) {
                            const uint4 *xv = (const uint4 *)(L.xs + ((size_t)tb * G + g) * kXPad);
#pragma unroll
                            for (int q = 0; q < 8; ++q) {
                                const uint4 xx = xv[q];
                                xl_[4 * q + 0] = xx.x;
                                xl_[4 * q + 1] = xx.y;
                                xl_[4 * q + 2] = xx.z;
                                xl_[4 * q + 3] = xx.w;
                            }
                        }
                        const uint32_t(&xp)[32] = pick_x<XREG>(xr_a[XREG ? tb * NG + gi : 0], xl_);
                        if constexpr (BITS != 2) {
                            float xq;
                            if constexpr (BF16)
                                xq = group_xq_bits_bf16<BITS>(cq[p][gi], xp, xg_a[tb][gi], a.dec_one);
                            else
                                xq = group_xq_bits_f16<BITS>(cq[p][gi], xp);
                            part[tb][pg] += s * (xq - z * xg_a[tb][gi]);
                        } else if constexpr (BF16) {
                            const float sp = group_dot<BF16>(pw, xp);
                            part[tb][pg] += s * (4.0f * sp - (4.0f + z) * xg_a[tb][gi]);
                        } else {
                            part[tb][pg] += s * (group_xq_f16(cq[p][gi].v, xp) - z * xg_a[tb][gi]);
                        }
                    }
                }
            }
            const int base = p0 + p - pg;           // first pass of this group
            if (pg == PRED - 1 && base < passes) {
                constexpr int LOGPRED = Log2<PRED>::v;
                const int psel = go >> (LOGSEG - LOGPRED);    // pass this lane ends up with
                const bool writer = (go & ((SEG / PRED) - 1)) == 0;
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const float v = transposed_reduce<PRED, SEG>(part[tb], lane);
                    const int r = (base + psel) * ROWS_PASS + wave * RPW + rs;
                    if (writer && r < nrows && tb < nt && base + psel < passes) {
                        L.vs[tb * cpw + r] = v;
                        L.mk[tb * cpw + r] = fabsf(v) > thr ? 1 : 0;
                    }
                }
            }
        }
    }
#undef LOAD_SLOT
#undef LOAD_PASS
    __syncthreads();

    // exports
    if (a.v_out || a.mask_out) {
        for (int i = tid; i < nt * nrows; i += THREADS) {
            const int tb = i / nrows, r = i - tb * nrows;
            const int t = L.tok_t[tb];
            if (a.layer) {
                if (a.mask_out)
                    a.mask_out[((size_t)t * (a.k + a.S) + L.tok_slot[tb]) * f + j0 + r] =
                        L.mk[tb * cpw + r];
            } else {
                if (a.mask_out) a.mask_out[(size_t)t * f + j0 + r] = L.mk[tb * cpw + r];
                if (a.v_out) a.v_out[(size_t)t * f + j0 + r] = L.vs[tb * cpw + r];
            }
        }
    }

    // ---- B: compaction of the union mask -------------------------------
    if (wave == 0) {
        int n = 0;
        for (int r0 = 0; r0 < nrows; r0 += 64) {
            const int r = r0 + lane;
            int on = 0;
            if (r < nrows)
                for (int tb = 0; tb < nt; ++tb) on |= L.mk[tb * cpw + r];
            const uint64_t bal = __ballot(on);
            const int pre = __popcll(bal & ((1ull << lane) - 1ull));
            if (on) L.list[n + pre] = (uint16_t)r;
            n += __popcll(bal);
        }
        if (lane == 0) L.misc[0] = n;
    }
    __syncthreads();
    const int n_act = L.misc[0];

    // ---- C: gate / down gathers over the active channels -----------------
    float yacc[TB][NCH][8];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int i = 0; i < NCH; ++i)
#pragma unroll
            for (int q = 0; q < 8; ++q) yacc[tb][i][q] = 0.f;

    if (n_act > 0) {
        uint4 xr[TB][NCH];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const int c = min(tid + THREADS * i, CPR - 1);
                xr[tb][i] = *(const uint4 *)(L.xs + ((size_t)tb * G + (c >> 3)) * kXPad + (c & 7) * 8);
                if (tid + THREADS * i >= CPR) xr[tb][i] = make_uint4(0, 0, 0, 0);
            }
        // h = SiLU(g) v of (token tb, list entry B0 + q) for lane tb * RB + q: the
        // wave partials of the gate dot are added in wave order
        auto lane_h = [&](int b0, int ln, const Lds &Ls, int nact, int ntok, int cp) -> float {
            float h = 0.f;
            if (ln < TB * RB) {
                const int tb = ln / RB, q = ln - tb * RB;
                const int ent = b0 + q;
                if (ent < nact && tb < ntok) {
                    const int r = (int)Ls.list[ent];
                    if (Ls.mk[tb * cp + r]) {
                        float g = 0.f;
#pragma unroll
                        for (int w = 0; w < W; ++w) g += Ls.gp[w * TB * RB + tb * RB + q];
                        h = silu(g) * Ls.vs[tb * cp + r];
                    }
                }
            }
            return h;
        };
        // loads of the batch of rows starting at list entry B0.  One token:
        // none past the list (a uniform branch per row; its single batch in
        // flight is waited for whole).  Several tokens: issued on every path,
        // an entry past the list reading zeros with no memory access, so the
        // count of loads in flight is the same on every path and the wait
        // before a batch's use leaves the next batch's loads in flight.
        const __amdgpu_buffer_rsrc_t rg = tile_rsrc(gate, (uint32_t)nrows * (uint32_t)d * 2u);
        const __amdgpu_buffer_rsrc_t rdn = tile_rsrc(down, (uint32_t)nrows * (uint32_t)d * 2u);
        uint32_t coff[NCH];                         // this thread's 16-byte piece of a row
#pragma unroll
        for (int i = 0; i < NCH; ++i) coff[i] = (uint32_t)min(tid + THREADS * i, CPR - 1);
#define C_LOAD(B0, GW, DW, ROWS)                                                               \
    _Pragma("unroll") for (int q = 0; q < RB; ++q) {                                           \
        const int ent = min((B0) + q, n_act - 1);                                              \
        ROWS[q] = (int)L.list[ent];                                                            \
        const bool okq = (B0) + q < n_act;          /* uniform */                              \
        _Pragma("unroll") for (int i = 0; i < NCH; ++i) {                                      \
            if constexpr (TB == 1) {                                                           \
                GW[q][i] = make_uint4(0, 0, 0, 0);                                             \
                DW[q][i] = make_uint4(0, 0, 0, 0);                                             \
                if (okq) {                                                                     \
                    GW[q][i] = row_load_nt(gate + (size_t)ROWS[q] * d + (size_t)coff[i] * 8);  \
                    DW[q][i] = row_load_nt(down + (size_t)ROWS[q] * d + (size_t)coff[i] * 8);  \
                }                                                                              \
            } else {                                                                           \
                const uint32_t off =                                                           \
                    okq ? ((uint32_t)ROWS[q] * (uint32_t)d + coff[i] * 8u) * 2u : kOob;        \
                GW[q][i] = row_bload(rg, off);                                                 \
                DW[q][i] = row_bload(rdn, off);                                                \
            }                                                                                  \
        }                                                                                      \
    }
        // gate dots of the batch, reduced over the wave and then over the waves
        // in LDS; h = SiLU(g) v per token and row; h * down into the slices of y
#define C_COMPUTE(B0, GW, DW, ROWS)                                                            \
    {                                                                                          \
        float p[TB * RB];                                                                      \
        _Pragma("unroll") for (int tb = 0; tb < TB; ++tb)                                      \
            _Pragma("unroll") for (int q = 0; q < RB; ++q) {                                   \
                float acc = 0.f;                                                               \
                _Pragma("unroll") for (int i = 0; i < NCH; ++i) {                              \
                    acc = dot2<BF16>(GW[q][i].x, xr[tb][i].x, acc);                            \
                    acc = dot2<BF16>(GW[q][i].y, xr[tb][i].y, acc);                            \
                    acc = dot2<BF16>(GW[q][i].z, xr[tb][i].z, acc);                            \
                    acc = dot2<BF16>(GW[q][i].w, xr[tb][i].w, acc);                            \
                }                                                                              \
                p[tb * RB + q] = acc;                                                          \
            }                                                                                  \
        {                                                                                      \
            constexpr int NP = TB * RB;                                                        \
            constexpr int NPR = NP < 64 ? NP : 64;                                             \
            static_assert(NP <= 64, "too many gate partials per batch");                       \
            const float v = transposed_reduce<NPR, 64>(p, lane);                               \
            constexpr int LOGNP = Log2<NPR>::v;                                                \
            const int idx = lane >> (6 - LOGNP);                                               \
            if ((lane & ((64 / NPR) - 1)) == 0) L.gp[wave * NP + idx] = v;                     \
        }                                                                                      \
        __syncthreads();                                                                       \
        /* h of (token tb, row q) is computed once, by lane tb * RB + q of every     */        \
        /* wave, and read from that lane by all (one v_readlane per row and token)    */        \
        const float hl = lane_h((B0), lane, L, n_act, nt, cpw);                                \
        _Pragma("unroll") for (int q = 0; q < RB; ++q) {                                       \
            _Pragma("unroll") for (int tb = 0; tb < TB; ++tb) {                                \
                const float h = __int_as_float(                                                \
                    __builtin_amdgcn_readlane(__float_as_int(hl), tb * RB + q));               \
                _Pragma("unroll") for (int i = 0; i < NCH; ++i) {                              \
                    const uint32_t dv[4] = {DW[q][i].x, DW[q][i].y, DW[q][i].z, DW[q][i].w};   \
                    _Pragma("unroll") for (int m = 0; m < 4; ++m) {                            \
                        yacc[tb][i][2 * m] += h * lo16_to_float<BF16>(dv[m]);                  \
                        yacc[tb][i][2 * m + 1] += h * hi16_to_float<BF16>(dv[m]);              \
                    }                                                                          \
                }                                                                              \
            }                                                                                  \
        }                                                                                      \
        __syncthreads();                                                                       \
    }
        uint4 gw[RB][NCH], dw[RB][NCH];
        int rows[RB];
        // bf16 at 512 threads has no room for a second set of rows (it spills)
        constexpr bool PIPE = TB > 1 && !(BF16 && THREADS >= 512);
        if constexpr (PIPE) {
            // two batches in flight: the next batch's rows load while this one
            // is multiplied (sets a and b alternate)
            uint4 gb[RB][NCH], db[RB][NCH];
            int rowsb[RB];
            // (a batch past the list issues loads that touch no memory)
            C_LOAD(0, gw, dw, rows)
            for (int b0 = 0; b0 < n_act; b0 += 2 * RB) {
                C_LOAD(b0 + RB, gb, db, rowsb)
                C_COMPUTE(b0, gw, dw, rows)
                if (b0 + RB >= n_act) break;
                C_LOAD(b0 + 2 * RB, gw, dw, rows)
                C_COMPUTE(b0 + RB, gb, db, rowsb)
            }
        } else {
            for (int b0 = 0; b0 < n_act; b0 += RB) {
                C_LOAD(b0, gw, dw, rows)
                C_COMPUTE(b0, gw, dw, rows)
            }
        }
#undef C_LOAD
#undef C_COMPUTE
    }
    // ---- D: this workgroup's scaled partial rows -------------------------
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        if (tb >= nt) continue;
        const float sc = L.tok_sc[tb];
        const int pstride = a.part_stride > 0 ? a.part_stride : a.tiles;
        float *dst = a.part + ((size_t)L.tok_row[tb] * pstride + tile) * d;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = tid + THREADS * i;
            if (c >= CPR) continue;
            float4 lo = make_float4(sc * yacc[tb][i][0], sc * yacc[tb][i][1],
                                    sc * yacc[tb][i][2], sc * yacc[tb][i][3]);
            float4 hi = make_float4(sc * yacc[tb][i][4], sc * yacc[tb][i][5],
                                    sc * yacc[tb][i][6], sc * yacc[tb][i][7]);
            // streamed: the reduce kernel reads each partial row once
            typedef float v4f __attribute__((ext_vector_type(4)));
            __builtin_nontemporal_store(v4f{lo.x, lo.y, lo.z, lo.w}, (v4f *)(dst + (size_t)c * 8));
            __builtin_nontemporal_store(v4f{hi.x, hi.y, hi.z, hi.w}, (v4f *)(dst + (size_t)c * 8 + 4));
        }
    }
}

// The kernel instance for this call: straight-line (ONE, PBX) or loop form;
// ROUTE: single-token layer calls that route inside the kernel (a separate
// instance, so that the other calls' code is unchanged by it).
template <bool BF16, int TB, class GEO, bool ROUTE, int BITS>
const void *pick_kernel(const SparseArgs &a)
{
    constexpr int rows_pass = GEO::W * (64 / GEO::SEG);
    constexpr int pb = pass_block<TB, GEO, BITS>();
    const int passes = (a.cpw + rows_pass - 1) / rows_pass;
    const bool one = passes <= pb;
    // (the widest geometry, and several tokens with two groups per lane, keep
    // the loop form: their straight-line versions spill)
    if constexpr (GEO::NG < 4 && (TB == 1 || GEO::NG == 1)) {
        if (one) return (const void *)expert_kernel<BF16, TB, GEO, true, 1, ROUTE, BITS>;
    }
    if constexpr (BITS == 2 && TB == 1 && GEO::NG == 1 && 2 * pb <= GEO::SEG) {
        if (!one && passes <= 2 * pb)
            return (const void *)expert_kernel<BF16, TB, GEO, true, 2, ROUTE, BITS>;
    }
    return (const void *)expert_kernel<BF16, TB, GEO, false, 1, ROUTE, BITS>;
}

template <bool BF16, int TB, class GEO, int BITS>
hipError_t launch_tb(const SparseArgs &a, hipStream_t s)
{
    size_t off[12];
    const size_t lds = lds_layout(a.d, a.cpw, TB, GEO::W, rows_per_batch<TB, GEO::NCH>(), off,
                                  a.route ? route_lds(a.E, a.k) : 0);
    const void *kern;
    if constexpr (TB == 1 && BITS == 2) {
        kern = a.route ? pick_kernel<BF16, TB, GEO, true, BITS>(a)
                       : pick_kernel<BF16, TB, GEO, false, BITS>(a);
    } else {
        if (a.route) return hipErrorInvalidValue;       // inline routing: one token, INT2
        kern = pick_kernel<BF16, TB, GEO, false, BITS>(a);
    }
    SparseArgs args = a;
    args.dec_mask = decode_const<BF16>().mask;
    args.dec_one = decode_const<BF16>().one;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    void *kargs[] = {(void *)&args};
    hipError_t e = hipLaunchKernel(kern, dim3(a.slots * a.tiles), dim3(GEO::THREADS), kargs, lds, s);
    if (e == hipSuccess) e = hipGetLastError();
    return e;
}

template <bool BF16, class GEO, int BITS>
hipError_t launch_geo(const SparseArgs &a, int tb, hipStream_t s)
{
    switch (tb) {
    case 1: return launch_tb<BF16, 1, GEO, BITS>(a, s);
    case 2:
        if constexpr (GEO::NG <= 2) return launch_tb<BF16, 2, GEO, BITS>(a, s);
        break;
    case 4:
        if constexpr (GEO::NG == 1) return launch_tb<BF16, 4, GEO, BITS>(a, s);
        break;
    default: break;
    }
    return hipErrorInvalidValue;
}

// Geometry by hidden size: see Geo.  Other code widths: d = 512 ... 4096.
// The smallest geometry whose SEG x NG groups and THREADS x NCH 16-byte
// chunks cover d (d % 64 == 0); lanes past the G = d / 64 groups read zeros,
// threads past the d / 8 chunks of a row hold none.
template <bool BF16, int BITS = 2>
hipError_t launch_dtype(const SparseArgs &a, int tb, hipStream_t s)
{
    if (a.d < 64 || a.d % 64 != 0) return hipErrorInvalidValue;
    if constexpr (BITS != 2) {
        if (a.d < 512) return hipErrorInvalidValue;
        if (a.d <= 512) return launch_geo<BF16, Geo<8, 1, 1, 64>, BITS>(a, tb, s);
        if (a.d <= 1024) return launch_geo<BF16, Geo<16, 1, 1, 128>, BITS>(a, tb, s);
        if (a.d <= 2048) return launch_geo<BF16, Geo<32, 1, 1, 256>, BITS>(a, tb, s);
        if (a.d <= 4096) return launch_geo<BF16, Geo<64, 1, 1, 512>, BITS>(a, tb, s);
        return hipErrorInvalidValue;
    } else {
        if (a.d <= 64) return launch_geo<BF16, Geo<1, 1, 1, 64>, 2>(a, tb, s);
        if (a.d <= 128) return launch_geo<BF16, Geo<2, 1, 1, 64>, 2>(a, tb, s);
        if (a.d <= 256) return launch_geo<BF16, Geo<4, 1, 1, 64>, 2>(a, tb, s);
        if (a.d <= 512) return launch_geo<BF16, Geo<8, 1, 1, 64>, 2>(a, tb, s);
        if (a.d <= 1024) return launch_geo<BF16, Geo<16, 1, 1, 128>, 2>(a, tb, s);
        if (a.d <= 2048) return launch_geo<BF16, Geo<32, 1, 1, 256>, 2>(a, tb, s);
        if (a.d <= 4096) return launch_geo<BF16, Geo<64, 1, 1, 512>, 2>(a, tb, s);
        if (a.d <= 8192) return launch_geo<BF16, Geo<64, 2, 2, 512>, 2>(a, tb, s);
        if (a.d <= 16384) return launch_geo<BF16, Geo<64, 4, 4, 512>, 2>(a, tb, s);
        return hipErrorInvalidValue;
    }
}

}  // namespace sparse
}  // namespace moeffn
