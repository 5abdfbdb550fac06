// Device check of routing data (moe_check_routing), for gfx950.
//
// The grouped calls take the routing as device arrays and trust them: split
// sizes that sum to the grouped row count, grouped rows and tokens in range,
// and a dest_row / src_token pair that describe one permutation, with each
// pick inside its expert's rows.  The routing is what sends each token to a
// few experts and groups the rows per expert [AutoModel page, section on the
// pain points of MoE fine-tuning; BioNeMo MoE recipe page, section
// GroupedLinear: the per-expert token counts].  This pass checks all of it
// on the device and ORs one bit per kind of violation into a status word, so
// that a caller can verify routing it built itself without a host copy of it.
#include "moe_mi355x.h"

#include "common.hpp"
#include "kernels.hpp"
#include "trace.hpp"

namespace moe {

__global__ void check_clear_kernel(int32_t* status) { *status = 0; }

// Grid-stride over the picks (t, j) and, for src_token, over the grouped rows;
// workgroup 0 also checks the split sizes.  Each workgroup ORs its bits into
// LDS and issues at most one global atomic.
__global__ __launch_bounds__(256) void check_routing_kernel(
    const int32_t* __restrict__ split, int E, int64_t rows, const int32_t* __restrict__ dest_row,
    const int32_t* __restrict__ src_token, const int32_t* __restrict__ topk_expert, int64_t T,
    int k, int32_t* status) {
    __shared__ int64_t off[65];     // expert row offsets (exclusive prefix of the sizes)
    __shared__ int bits_lds;
    const int tid = threadIdx.x;
    int bits = 0;
    if (tid == 0) bits_lds = 0;
    if (tid < 64) {
        const int64_t n = (split && tid < E) ? split[tid] : 0;
        int64_t incl = n;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int64_t t = __shfl_up(incl, o);
            if (tid >= o) incl += t;
        }
        off[tid] = incl - n;
        if (tid == 63) off[64] = incl;
        if (blockIdx.x == 0 && split) {
            if (n < 0) bits |= MOE_CHECK_SPLIT_NEGATIVE;
            if (tid == 63 && incl != rows) bits |= MOE_CHECK_SPLIT_SUM;
        }
    }
    __syncthreads();
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t picks = dest_row ? T * k : 0;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + tid; i < picks; i += stride) {
        const int64_t t = i / k;
        const int64_t d = dest_row[i];
        const bool d_ok = d >= 0 && d < rows;
        if (!d_ok) bits |= MOE_CHECK_DEST_RANGE;
        if (d_ok && src_token && src_token[d] != t) bits |= MOE_CHECK_MISMATCH;
        if (topk_expert) {
            const int e = topk_expert[i];
            if (e < 0 || e >= E) {
                bits |= MOE_CHECK_EXPERT_RANGE;
            } else if (d_ok && split && (d < off[e] || d >= off[e + 1])) {
                bits |= MOE_CHECK_MISMATCH;   // the pick's row is outside its expert's rows
            }
        }
    }
    const int64_t nsrc = src_token ? rows : 0;
    for (int64_t r = (int64_t)blockIdx.x * blockDim.x + tid; r < nsrc; r += stride) {
        const int64_t s = src_token[r];
        if (s < 0 || s >= T) bits |= MOE_CHECK_SRC_RANGE;
    }
    if (bits) atomicOr(&bits_lds, bits);
    __syncthreads();
    if (tid == 0 && bits_lds) atomicOr(status, bits_lds);
}

hipError_t launch_check_routing(const int32_t* split, int E, int64_t rows,
                                const int32_t* dest_row, const int32_t* src_token,
                                const int32_t* topk_expert, int64_t T, int k, int32_t* status,
                                hipStream_t s) {
    TraceScope ts("check_routing", s);
    // a kernel, not a memset, clears the word (safe under graph capture)
    check_clear_kernel<<<1, 1, 0, s>>>(status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = (dest_row ? T * k : 0) > rows ? T * k : rows;
    int64_t blocks = (n + 255) / 256;
    blocks = blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks);
    check_routing_kernel<<<(unsigned)blocks, 256, 0, s>>>(split, E, rows, dest_row, src_token,
                                                          topk_expert, T, k, status);
    return hipGetLastError();
}

}  // namespace moe
