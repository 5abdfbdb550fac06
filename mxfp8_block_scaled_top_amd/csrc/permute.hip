// Dispatch (permute) and combine (unpermute) of token rows, for gfx950.
//
// Tokens are sent to the experts that compute them and the results are sent
// back [AutoModel page, section on expert parallelism]; on one GPU the
// "sending" is a row copy into the expert-grouped order that the grouped GEMM
// consumes [BioNeMo MoE recipe page, section GroupedLinear].
//
// Grouped rows outside [0, T*k) in dest_row are skipped, so routing that does
// not hold the preconditions gives unspecified rows but no access outside the
// buffers.
//
// Both kernels are HBM-bound row copies: one thread moves one 16-byte chunk
// (8 bf16) so every wave reads and writes whole 1 KiB row segments.  Permute
// reads each token row once and writes it to its k grouped rows (the minimum
// traffic: T*H*2 read + T*k*H*2 written); unpermute reads the k grouped rows
// of a token and writes the fp32 sum once, rounded to bf16.
#include "common.hpp"
#include "kernels.hpp"
#include "trace.hpp"

namespace moe {

__global__ __launch_bounds__(256) void permute_kernel(const u32x4* __restrict__ x, int T, int cpr,
                                                      int k, const int32_t* __restrict__ dest_row,
                                                      const float* __restrict__ topk_prob,
                                                      u32x4* __restrict__ xp,
                                                      float* __restrict__ prob_perm) {
    const size_t total = (size_t)T * cpr;
    const int64_t rows = (int64_t)T * k;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (size_t)gridDim.x * blockDim.x) {
        size_t t = i / cpr;
        int c = (int)(i - t * cpr);
        u32x4 v = __builtin_nontemporal_load(x + i);
        const int32_t* d = dest_row + t * k;
        for (int j = 0; j < k; ++j) {
            const int r = d[j];
            if ((unsigned)r >= (unsigned)rows) continue;   // out of range: dropped
            xp[(size_t)r * cpr + c] = v;
            if (c == 0 && prob_perm) prob_perm[r] = topk_prob[t * k + j];
        }
    }
}

// The probabilities alone (the rows are gathered by their consumer).
__global__ __launch_bounds__(256) void permute_prob_kernel(int64_t picks,
                                                           const int32_t* __restrict__ dest_row,
                                                           const float* __restrict__ topk_prob,
                                                           float* __restrict__ prob_perm) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < picks && (uint64_t)(uint32_t)dest_row[i] < (uint64_t)picks)
        prob_perm[dest_row[i]] = topk_prob[i];
}

__global__ __launch_bounds__(256) void unpermute_kernel(const u32x4* __restrict__ yp, int T,
                                                        int cpr, int k,
                                                        const int32_t* __restrict__ dest_row,
                                                        const float* __restrict__ topk_prob,
                                                        u32x4* __restrict__ y) {
    const size_t total = (size_t)T * cpr;
    const int64_t rows = (int64_t)T * k;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (size_t)gridDim.x * blockDim.x) {
        size_t t = i / cpr;
        int c = (int)(i - t * cpr);
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        const int32_t* d = dest_row + t * k;
        for (int j = 0; j < k; ++j) {
            if ((unsigned)d[j] >= (unsigned)rows) continue;   // out of range: adds nothing
            u32x4 v = yp[(size_t)d[j] * cpr + c];
            float w = topk_prob ? topk_prob[t * k + j] : 1.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (topk_prob) {
                    acc[2 * q] += w * lo_bf16(v[q]);
                    acc[2 * q + 1] += w * hi_bf16(v[q]);
                } else {
                    acc[2 * q] += lo_bf16(v[q]);
                    acc[2 * q + 1] += hi_bf16(v[q]);
                }
            }
        }
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
        y[i] = o;
    }
}

static unsigned grid_for(size_t n, int threads) {
    size_t b = (n + threads - 1) / threads;
    size_t cap = 256 * 64;                  // 64 blocks per CU is plenty for a copy
    return (unsigned)(b < cap ? (b ? b : 1) : cap);
}

hipError_t launch_permute(const bf16_t* x, int T, int H, int k, const int32_t* dest_row,
                          const float* topk_prob, bf16_t* xp, float* prob_perm,
                          hipStream_t s) {
    size_t n = (size_t)T * (H / 8);
    if (n == 0) return hipSuccess;
    if (!x) {   // probabilities only
        const int64_t picks = (int64_t)T * k;
        TraceScope ts("permute_prob", s);
        permute_prob_kernel<<<(unsigned)((picks + 255) / 256), 256, 0, s>>>(picks, dest_row,
                                                                            topk_prob, prob_perm);
        return hipGetLastError();
    }
    TraceScope ts("permute", s);
    permute_kernel<<<grid_for(n, 256), 256, 0, s>>>((const u32x4*)x, T, H / 8, k, dest_row,
                                                    topk_prob, (u32x4*)xp,
                                                    topk_prob ? prob_perm : nullptr);
    return hipGetLastError();
}

hipError_t launch_unpermute(const bf16_t* yp, int T, int H, int k, const int32_t* dest_row,
                            const float* topk_prob, bf16_t* y, hipStream_t s) {
    size_t n = (size_t)T * (H / 8);
    if (n == 0) return hipSuccess;
    TraceScope ts("unpermute", s);
    unpermute_kernel<<<grid_for(n, 256), 256, 0, s>>>((const u32x4*)yp, T, H / 8, k, dest_row,
                                                      topk_prob, (u32x4*)y);
    return hipGetLastError();
}

}  // namespace moe
