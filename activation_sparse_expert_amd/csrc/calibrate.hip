// Threshold calibration on the GPU: t = the q-quantile of |v| over n values
// (FloE review, "高效稀疏 GEMV 内核": t_ij is a per-expert threshold that sets
// the activation sparsity; the pages leave its placement open, and the
// library's reading is the linear-interpolation quantile of |v| over
// calibration tokens).
//
// The two order statistics the interpolation needs (ranks lo and hi) are
// found by a radix select on the bit patterns of |v|: non-negative floats
// order like their 31-bit patterns.  Three passes take 11, 10 and 10 bits;
// in each, every workgroup builds LDS histograms of the digit of the values
// that match each rank's prefix so far and adds them into global bins, and
// one workgroup then finds the bin holding each rank, narrows the prefix and
// clears the bins for the next pass.  The last pass interpolates in fp64 as
// the oracle's quantile does and rounds to fp32.
#include "device.hpp"
#include "internal.hpp"

namespace moeffn {

namespace {

constexpr int kCalThreads = 256;
constexpr int kFindThreads = 1024;
constexpr int kMaxBins = 2048;

struct PassGeo {
    int shift, bits;                    // digit = (u >> shift) & ((1 << bits) - 1)
};
__host__ __device__ constexpr PassGeo pass_geo(int pass)
{
    return pass == 0 ? PassGeo{20, 11} : (pass == 1 ? PassGeo{10, 10} : PassGeo{0, 10});
}

// state[j] = {prefix of rank j's value above this pass's digit, rank within it}
__global__ void __launch_bounds__(kCalThreads)
cal_hist_kernel(const float *v, long long n, int pass, const int32_t *state, int32_t *ghist)
{
    __shared__ int32_t h[2][kMaxBins];
    const PassGeo g = pass_geo(pass);
    const int nb = 1 << g.bits;
    for (int i = threadIdx.x; i < 2 * kMaxBins; i += kCalThreads) (&h[0][0])[i] = 0;
    const uint32_t p0 = pass == 0 ? 0u : (uint32_t)state[0];
    const uint32_t p1 = pass == 0 ? 0u : (uint32_t)state[2];
    const int top = g.shift + g.bits;    // bits above the digit form the prefix
    __syncthreads();
    const long long stride = (long long)gridDim.x * kCalThreads;
    for (long long i = (long long)blockIdx.x * kCalThreads + threadIdx.x; i < n; i += stride) {
        const uint32_t u = __float_as_uint(v[i]) & 0x7FFFFFFFu;
        const uint32_t dig = (u >> g.shift) & (uint32_t)(nb - 1);
        const uint32_t pre = top >= 31 ? 0u : (u >> top);
        if (pre == p0) atomicAdd(&h[0][dig], 1);
        if (pre == p1) atomicAdd(&h[1][dig], 1);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nb; i += kCalThreads) {
        if (h[0][i]) atomicAdd(&ghist[i], h[0][i]);
        if (h[1][i]) atomicAdd(&ghist[kMaxBins + i], h[1][i]);
    }
}

// One workgroup: for each rank, the bin whose running count passes it; the
// prefix gains that digit and the rank drops the counts below it.  The bins
// are cleared for the next pass.  After the last pass the prefixes are the
// two values, combined as a + (b - a) g, or b - (b - a)(1 - g) from g = 1/2.
__global__ void __launch_bounds__(kFindThreads)
cal_find_kernel(int pass, long long r_lo, long long r_hi, double gamma, int32_t *state,
                int32_t *ghist, float *out)
{
    __shared__ int32_t sums[kFindThreads];
    __shared__ int32_t pick[2][2];
    const PassGeo g = pass_geo(pass);
    const int nb = 1 << g.bits;
    const int per = (nb + kFindThreads - 1) / kFindThreads;     // bins per thread (1 or 2)
    const int tid = threadIdx.x;
    for (int j = 0; j < 2; ++j) {
        const int32_t rank = pass == 0 ? (int32_t)(j == 0 ? r_lo : r_hi) : state[2 * j + 1];
        int32_t *hj = ghist + j * kMaxBins;
        int32_t c[2] = {0, 0};
        int32_t own = 0;
        for (int b = 0; b < per; ++b) {
            const int bin = tid * per + b;
            c[b] = bin < nb ? hj[bin] : 0;
            own += c[b];
        }
        sums[tid] = own;
        __syncthreads();
        // inclusive scan of the per-thread counts (Hillis-Steele in LDS)
        for (int off = 1; off < kFindThreads; off <<= 1) {
            const int32_t add = tid >= off ? sums[tid - off] : 0;
            __syncthreads();
            sums[tid] += add;
            __syncthreads();
        }
        const int32_t before = sums[tid] - own;
        int32_t run = before;
        for (int b = 0; b < per; ++b) {
            if (run <= rank && rank < run + c[b]) {
                pick[j][0] = tid * per + b;         // exactly one thread's bin holds the rank
                pick[j][1] = rank - run;
            }
            run += c[b];
        }
        __syncthreads();
        for (int b = 0; b < per; ++b) {
            const int bin = tid * per + b;
            if (bin < nb) hj[bin] = 0;             // cleared for the next pass
        }
        __syncthreads();
    }
    if (tid == 0) {
        for (int j = 0; j < 2; ++j) {
            const uint32_t pre = pass == 0 ? 0u : (uint32_t)state[2 * j];
            state[2 * j] = (int32_t)((pre << g.bits) | (uint32_t)pick[j][0]);
            state[2 * j + 1] = pick[j][1];
        }
        if (pass == 2) {
            const double a = (double)__uint_as_float((uint32_t)state[0]);
            const double b = (double)__uint_as_float((uint32_t)state[2]);
            const double diff = b - a;
            const double r = gamma >= 0.5 ? b - diff * (1.0 - gamma) : a + diff * gamma;
            *out = (float)r;
        }
    }
}

}  // namespace

size_t calibrate_ws_bytes() { return (size_t)2 * kMaxBins * 4 + 64; }

hipError_t launch_calibrate(const float *v, long long n, long long r_lo, long long r_hi,
                            double gamma, float *out, void *ws, hipStream_t s)
{
    int32_t *ghist = (int32_t *)ws;
    int32_t *state = ghist + 2 * kMaxBins;
    hipError_t e = launch_fill_zero(ws, calibrate_ws_bytes(), s);
    if (e != hipSuccess) return e;
    long long blocks = (n + kCalThreads * 8 - 1) / (kCalThreads * 8);
    if (blocks > 1024) blocks = 1024;
    if (blocks < 1) blocks = 1;
    for (int pass = 0; pass < 3; ++pass) {
        hipLaunchKernelGGL(cal_hist_kernel, dim3((unsigned)blocks), dim3(kCalThreads), 0, s, v, n,
                           pass, (const int32_t *)state, ghist);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(cal_find_kernel, dim3(1), dim3(kFindThreads), 0, s, pass, r_lo, r_hi,
                           gamma, state, ghist, out);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace moeffn
