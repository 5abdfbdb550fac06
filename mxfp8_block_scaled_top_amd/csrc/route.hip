// Top-k routing, per-expert counts (split_sizes) and the stable grouped-row
// permutation, for gfx950.
//
// Each token goes to a few experts only [AutoModel page, section on the pain
// points of MoE fine-tuning: sparse activation]; the grouped GEMM takes the
// rows of all experts in one call with the number of rows of each expert
// [BioNeMo MoE recipe page, section GroupedLinear].
//
// Three launches, all deterministic (integer atomics are not used):
//   1. route_topk:    one thread per token, its row of logits in registers.
//                     Picks the k largest fp32 logits (ties -> lower expert),
//                     softmax over the picks, and the token's rank among the
//                     block's earlier tokens that picked the same expert (wave
//                     ballots per expert, kept in LDS with per-wave counts).
//                     Writes per-block expert counts.
//   2. route_scan:    one wave.  Per expert, exclusive scan of the block counts
//                     (the blocks' base rows), split_sizes and offsets.
//   3. route_scatter: one thread per pick: dest_row and src_token.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"
#include "trace.hpp"

namespace moe {

constexpr int kRouteThreads = 256;          // tokens per block (4 waves)
constexpr int kRouteWaves = kRouteThreads / kWave;

__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, uint32_t flags,
    int32_t* __restrict__ topk_expert, float* __restrict__ topk_prob,
    int32_t* __restrict__ local_rank, int32_t* __restrict__ block_counts) {
    __shared__ int wave_cnt[kRouteWaves][kMaxExperts];
    __shared__ uint64_t wave_bal[kRouteWaves][kMaxExperts];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int t = blockIdx.x * kRouteThreads + tid;
    const bool valid = t < T;

    uint64_t picked = 0;
    if (valid) {
        const float* row = logits + (size_t)t * E;
        int32_t* sel = topk_expert + (size_t)t * k;
        float* prob = topk_prob + (size_t)t * k;
        // the row in registers (E <= kMaxExperts; E is uniform, so the tests
        // below are scalar branches, and entries e >= E are neither loaded
        // nor used)
        float v[kMaxExperts];
#pragma unroll
        for (int e = 0; e < kMaxExperts; ++e) {
            if (e < E) v[e] = row[e];
            else v[e] = 0.f;
        }
        // k scans: strict '>' keeps the lowest index among equals.  The picked
        // logits go to prob[] until the denominator is known.
        float top = 0.f, denom = 0.f;
        for (int j = 0; j < k; ++j) {
            float bv = 0.f;
            int be = -1;
#pragma unroll
            for (int e = 0; e < kMaxExperts; ++e) {
                if (e < E && !((picked >> e) & 1ull) && (be < 0 || v[e] > bv)) {
                    bv = v[e];
                    be = e;
                }
            }
            picked |= 1ull << be;
            sel[j] = be;
            prob[j] = bv;
            if (j == 0) top = bv;
            denom += expf(bv - top);
        }
        if (flags & 1u) {
            // softmax over all experts, taken at the picks
            float mx = top;                  // the first pick is the row maximum
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < kMaxExperts; ++e)
                if (e < E) s += expf(v[e] - mx);
            for (int j = 0; j < k; ++j) prob[j] = expf(prob[j] - mx) / s;
        } else {
            for (int j = 0; j < k; ++j) prob[j] = expf(prob[j] - top) / denom;
        }
    }

    // Per-wave ballots and counts of each expert, then the block-level prefix
    // over waves.
    for (int e = 0; e < E; ++e) {
        uint64_t bal = __ballot((picked >> e) & 1ull);
        if (lane == 0) {
            wave_bal[wave][e] = bal;
            wave_cnt[wave][e] = __popcll(bal);
        }
    }
    __syncthreads();
    if (tid < E) {
        int run = 0;
        for (int w = 0; w < kRouteWaves; ++w) {
            int c = wave_cnt[w][tid];
            wave_cnt[w][tid] = run;          // exclusive prefix over waves
            run += c;
        }
        block_counts[(size_t)blockIdx.x * E + tid] = run;
    }
    __syncthreads();
    if (valid) {
        const uint64_t lt = lanemask_lt();
        for (int j = 0; j < k; ++j) {
            const int e = topk_expert[(size_t)t * k + j];
            local_rank[(size_t)t * k + j] = wave_cnt[wave][e] + __popcll(wave_bal[wave][e] & lt);
        }
    }
}

// One wave: lane e owns expert e.
__global__ __launch_bounds__(64) void route_scan_kernel(
    const int32_t* __restrict__ block_counts, int nblocks, int E,
    int32_t* __restrict__ block_base, int32_t* __restrict__ split_sizes,
    int32_t* __restrict__ expert_offsets) {
    const int e = threadIdx.x;
    int total = 0;
    if (e < E) {
        // (unrolled so that several loads are in flight at once)
#pragma unroll 8
        for (int b = 0; b < nblocks; ++b) total += block_counts[(size_t)b * E + e];
    }
    int incl = wave_incl_scan(e < E ? total : 0);
    int off = incl - (e < E ? total : 0);
    if (e < E) {
        split_sizes[e] = total;
        expert_offsets[e] = off;
        int run = off;
#pragma unroll 8
        for (int b = 0; b < nblocks; ++b) {
            int c = block_counts[(size_t)b * E + e];
            block_base[(size_t)b * E + e] = run;
            run += c;
        }
    }
    if (e == E - 1) expert_offsets[E] = incl;
}

__global__ void route_scatter_kernel(const int32_t* __restrict__ topk_expert,
                                     const int32_t* __restrict__ local_rank,
                                     const int32_t* __restrict__ block_base, int T, int E, int k,
                                     int32_t* __restrict__ dest_row,
                                     int32_t* __restrict__ src_token) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)T * k) return;
    int t = (int)(i / k);
    int e = topk_expert[i];
    int row = block_base[(size_t)(t / kRouteThreads) * E + e] + local_rank[i];
    dest_row[i] = row;
    src_token[row] = t;
}

// Backward of the routing probabilities; one thread per token.
__global__ void route_bwd_kernel(const float* __restrict__ topk_prob,
                                 const float* __restrict__ dprob_perm,
                                 const int32_t* __restrict__ dest_row,
                                 const int32_t* __restrict__ topk_expert,
                                 const float* __restrict__ logits, int T, int E, int k,
                                 uint32_t flags, float* __restrict__ dlogits) {
    int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T) return;
    const size_t base = (size_t)t * k;
    float* out = dlogits + (size_t)t * E;
    const unsigned rows = (unsigned)T * (unsigned)k;
    // a grouped row outside [0, T*k) reads gradient 0; an expert outside
    // [0, E) receives nothing (routing that breaks the preconditions gives
    // unspecified values, never an access outside the buffers)
    auto dp = [&](int j) -> float {
        const unsigned r = (unsigned)dest_row[base + j];
        return r < rows ? dprob_perm[r] : 0.f;
    };
    auto ex = [&](int j) -> int {
        const int e = topk_expert[base + j];
        return (unsigned)e < (unsigned)E ? e : -1;
    };
    if (flags & 1u) {
        const float* row = logits + (size_t)t * E;
        float mx = row[0];
        for (int e = 1; e < E; ++e) mx = fmaxf(mx, row[e]);
        float s = 0.f;
        for (int e = 0; e < E; ++e) s += expf(row[e] - mx);
        float inv = 1.f / s;
        float dot = 0.f;
        for (int j = 0; j < k; ++j) {
            const int e = ex(j);
            if (e < 0) continue;
            float p = expf(row[e] - mx) * inv;
            dot += p * dp(j);
        }
        for (int e = 0; e < E; ++e) {
            float g = 0.f;
            for (int j = 0; j < k; ++j)
                if (ex(j) == e) g = dp(j);
            out[e] = expf(row[e] - mx) * inv * (g - dot);
        }
        return;
    }
    float dot = 0.f;
    for (int j = 0; j < k; ++j) dot += topk_prob[base + j] * dp(j);
    for (int e = 0; e < E; ++e) out[e] = 0.f;
    for (int j = 0; j < k; ++j) {
        const int e = ex(j);
        if (e < 0) continue;
        float p = topk_prob[base + j];
        out[e] = p * (dp(j) - dot);
    }
}

// Scratch of the no-allocation routing entry point: one static device array,
// which every GPU the library runs on holds (each at its own address) until
// the process ends.  Host code never passes `scratch` itself to a kernel (on
// the host it names a host-side stand-in): route_scratch() fetches the array's
// device address once per device, with that device current, and the kernels
// take that address like the caller's workspace of moe_route.
static __device__ __align__(256) uint8_t scratch[kRouteScratchBytes];

namespace {
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];
}  // namespace

hipError_t route_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev]() {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
    *ptr = g_scratch_ptr[dev];
    return *ptr ? hipSuccess : hipErrorInvalidSymbol;
}

size_t route_workspace_bytes(int64_t T, int E, int k) {
    size_t nb = (size_t)((T + kRouteThreads - 1) / kRouteThreads);
    size_t bytes = 2 * nb * (size_t)E * sizeof(int32_t)      // counts + bases
                   + (size_t)T * k * sizeof(int32_t);         // local ranks
    return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_route(const float* logits, int T, int E, int k, uint32_t flags,
                        int32_t* topk_expert, float* topk_prob, int32_t* split_sizes,
                        int32_t* expert_offsets, int32_t* dest_row, int32_t* src_token,
                        void* ws, hipStream_t s) {
    int nb = (T + kRouteThreads - 1) / kRouteThreads;
    int32_t* counts = (int32_t*)ws;
    int32_t* bases = counts + (size_t)nb * E;
    int32_t* ranks = bases + (size_t)nb * E;
    if (nb > 0) {
        TraceScope ts("route_topk", s);
        route_topk_kernel<<<nb, kRouteThreads, 0, s>>>(logits, T, E, k, flags, topk_expert,
                                                       topk_prob, ranks, counts);
    }
    {
        TraceScope ts("route_scan", s);
        route_scan_kernel<<<1, 64, 0, s>>>(counts, nb, E, bases, split_sizes, expert_offsets);
    }
    size_t n = (size_t)T * k;
    if (n > 0) {
        TraceScope ts("route_scatter", s);
        route_scatter_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
            topk_expert, ranks, bases, T, E, k, dest_row, src_token);
    }
    return hipGetLastError();
}

hipError_t launch_route_bwd(const float* topk_prob, const float* dprob_perm,
                            const int32_t* dest_row, const int32_t* topk_expert,
                            const float* logits, int T, int E, int k, uint32_t flags,
                            float* dlogits, hipStream_t s) {
    if (T > 0) {
        TraceScope ts("route_bwd", s);
        route_bwd_kernel<<<(T + 255) / 256, 256, 0, s>>>(topk_prob, dprob_perm, dest_row,
                                                         topk_expert, logits, T, E, k, flags,
                                                         dlogits);
    }
    return hipGetLastError();
}

}  // namespace moe
