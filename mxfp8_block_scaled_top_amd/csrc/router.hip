// Router linear layer in front of the top-k routing, for gfx950.
//
// Every token is routed to a few experts [AutoModel page, section on the pain
// points of MoE fine-tuning]; the routing logits are a bias-free linear map of
// the token's hidden state, logits = X W_r^T (X bf16 [T, H], W_r bf16 [E, H],
// fp32 accumulation).
//
//   router_logits  the contraction over H on the matrix cores (bf16 MFMA
//                  32x32x16): a workgroup owns 32 tokens and all E <= 64
//                  experts; its 8 waves take the 64-value K steps round robin
//                  and meet in LDS.  Each lane loads 64 contiguous bytes of its
//                  token row per K step (both halves of the wave: the row's
//                  whole 128 bytes), and the same K positions of the W_r row
//                  of its expert.  Reads X once: HBM-bound.
//   router_dx      backward to the tokens, fused with the combine of the
//                  expert path: dX[t] = bf16(sum_j dXp[dest_row[t][j]] +
//                  sum_e dlogits[t, e] W_r[e]) summed in fp32.  A workgroup
//                  owns 32 tokens x 256 columns with that slice of W_r and the
//                  tokens' dlogits in LDS; a thread owns 8 columns of 4 tokens.
//   router_dw      dW_r = dlogits^T X: fp32 partial sums over fixed token
//                  splits (a lane owns 4 columns for 16 experts at a time),
//                  then a reduction over the splits in split order into bf16.
//                  No atomics: the results do not depend on scheduling.
#include "common.hpp"
#include "kernels.hpp"
#include "trace.hpp"

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 rt_bf16x8;
typedef __attribute__((ext_vector_type(16))) float rt_f32x16;

constexpr int kRtTok = 32;          // tokens per logits workgroup
constexpr int kRtWaves = 8;         // waves per logits workgroup (K steps round robin)
constexpr int kDxTok = 32;          // tokens per dx workgroup
constexpr int kDxCols = 256;        // columns per dx / dw workgroup
constexpr int kDwExperts = 16;      // experts per dw register pass

__global__ __launch_bounds__(64 * kRtWaves) void router_logits_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w, int T, int H, int E,
    float* __restrict__ logits) {
    __shared__ float red[kRtWaves][kRtTok][65];
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    const int r = lane & 31, h = lane >> 5;
    const int t0 = blockIdx.x * kRtTok;
    // rows past T and experts past E load a valid row and are never stored
    const int64_t tr = min(t0 + r, T - 1);
    const bf16_t* xr = x + tr * H + 32 * h;
    const bf16_t* w0 = w + (int64_t)min(r, E - 1) * H + 32 * h;
    const bf16_t* w1 = w + (int64_t)min(32 + r, E - 1) * H + 32 * h;
    const bool two = E > 32;
    rt_f32x16 acc0, acc1;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc0[v] = acc1[v] = 0.f;
    // K step ks covers [64 ks, 64 ks + 64): lane half h holds [64 ks + 32 h,
    // +32) of its row as 4 chunks of 8; MFMA q pairs chunk q of the token row
    // with chunk q of the expert row (the same K positions on both sides).
    const int nks = H / 64;
    auto load = [&](int ks, u32x4 (&xa)[4], u32x4 (&wa)[4], u32x4 (&wb)[4]) {
        const int k0 = ks * 64;
#pragma unroll
        for (int q = 0; q < 4; ++q) xa[q] = *(const u32x4*)(xr + k0 + 8 * q);
#pragma unroll
        for (int q = 0; q < 4; ++q) wa[q] = *(const u32x4*)(w0 + k0 + 8 * q);
        if (two) {
#pragma unroll
            for (int q = 0; q < 4; ++q) wb[q] = *(const u32x4*)(w1 + k0 + 8 * q);
        }
    };
    auto mma = [&](const u32x4 (&xa)[4], const u32x4 (&wa)[4], const u32x4 (&wb)[4]) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(rt_bf16x8, xa[q]),
                                                          __builtin_bit_cast(rt_bf16x8, wa[q]),
                                                          acc0, 0, 0, 0);
        if (two) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(rt_bf16x8, xa[q]), __builtin_bit_cast(rt_bf16x8, wb[q]),
                    acc1, 0, 0, 0);
        }
    };
    // two of the wave's K steps per iteration, both loaded before either is
    // used (twice the bytes in flight)
    for (int ks = wave; ks < nks; ks += 2 * kRtWaves) {
        u32x4 xa[4], wa[4], wb[4], xb[4], va[4], vb[4];
        const bool second = ks + kRtWaves < nks;
        load(ks, xa, wa, wb);
        if (second) load(ks + kRtWaves, xb, va, vb);
        mma(xa, wa, wb);
        if (second) mma(xb, va, vb);
    }
    // accumulator v of lane (column c, half hi) is token row 8(v/4) + 4 hi + v%4
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int row = 8 * (v >> 2) + 4 * h + (v & 3);
        red[wave][row][r] = acc0[v];
        red[wave][row][32 + r] = two ? acc1[v] : 0.f;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kRtTok * E; i += 64 * kRtWaves) {
        const int row = i / E, e = i - row * E;
        if (t0 + row < T) {
            float sum = red[0][row][e];
#pragma unroll
            for (int q = 1; q < kRtWaves; ++q) sum += red[q][row][e];
            logits[(int64_t)(t0 + row) * E + e] = sum;
        }
    }
}

__global__ __launch_bounds__(256) void router_dx_kernel(const float* __restrict__ G,
                                                        const bf16_t* __restrict__ w,
                                                        const bf16_t* __restrict__ dxp,
                                                        const int32_t* __restrict__ dest_row,
                                                        int T, int H, int E, int k,
                                                        bf16_t* __restrict__ dx) {
    __shared__ u32x4 ws[kMaxExperts][kDxCols / 8];       // W_r[e][c0 + 8 cc .. +8], bf16
    __shared__ float gs[kDxTok][kMaxExperts + 1];
    const int tid = threadIdx.x;
    const int c0 = blockIdx.x * kDxCols, t0 = blockIdx.y * kDxTok;
    for (int i = tid; i < E * (kDxCols / 8); i += 256) {
        const int e = i / (kDxCols / 8), cc = i - e * (kDxCols / 8);
        const int c = c0 + 8 * cc;
        ws[e][cc] = c < H ? *(const u32x4*)(w + (int64_t)e * H + c) : (u32x4){0u, 0u, 0u, 0u};
    }
    for (int i = tid; i < kDxTok * E; i += 256) {
        const int tt = i / E, e = i - tt * E;
        gs[tt][e] = t0 + tt < T ? G[(int64_t)(t0 + tt) * E + e] : 0.f;
    }
    __syncthreads();
    const int cc = tid & 31, tg = tid >> 5;
    const int c = c0 + 8 * cc;
    if (c >= H) return;
    float acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[i][q] = 0.f;
    if (dxp) {
        // expert path, slots in order; two tokens and up to 8 slots at a time,
        // the grouped-row indices first, then all their rows, so that up to
        // 16 row loads are in flight
#pragma unroll
        for (int i0 = 0; i0 < 4; i0 += 2) {
            for (int j0 = 0; j0 < k; j0 += 8) {
                int64_t rows[2][8];
#pragma unroll
                for (int ii = 0; ii < 2; ++ii) {
                    const int t = t0 + tg + 8 * (i0 + ii);
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        rows[ii][u] = (t < T && j0 + u < k) ? dest_row[(int64_t)t * k + j0 + u] : -1;
#pragma unroll
                for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                    for (int u = 0; u < 8; ++u)   // outside [0, T*k): no row (skipped)
                        if (rows[ii][u] >= (int64_t)T * k) rows[ii][u] = -1;
                }
                u32x4 v[2][8];
#pragma unroll
                for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        v[ii][u] = rows[ii][u] >= 0 ? *(const u32x4*)(dxp + rows[ii][u] * H + c)
                                                    : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
                for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        if (rows[ii][u] < 0) continue;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            acc[i0 + ii][2 * q] += lo_bf16(v[ii][u][q]);
                            acc[i0 + ii][2 * q + 1] += hi_bf16(v[ii][u][q]);
                        }
                    }
            }
        }
    }
    for (int e = 0; e < E; ++e) {              // router path, experts in order
        const u32x4 wv = ws[e][cc];
        float wf[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            wf[2 * q] = lo_bf16(wv[q]);
            wf[2 * q + 1] = hi_bf16(wv[q]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float g = gs[tg + 8 * i][e];
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[i][q] = __builtin_fmaf(g, wf[q], acc[i][q]);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + tg + 8 * i;
        if (t < T)
            *(u32x4*)(dx + (int64_t)t * H + c) =
                (u32x4){pack_bf16x2(acc[i][0], acc[i][1]), pack_bf16x2(acc[i][2], acc[i][3]),
                        pack_bf16x2(acc[i][4], acc[i][5]), pack_bf16x2(acc[i][6], acc[i][7])};
    }
}

// part[s][e][c] = sum over the tokens of split s (wave w takes tokens
// w, w+4, .. of the split in ascending order; the 4 waves are then added in
// order).
__global__ __launch_bounds__(256) void router_dw_kernel(const float* __restrict__ G,
                                                        const bf16_t* __restrict__ x, int T,
                                                        int H, int E, int tps,
                                                        float* __restrict__ part) {
    __shared__ float red[4][kDwExperts][kDxCols + 4];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane((int)(tid >> 6));
    const int lane = tid & 63;
    const int cb = blockIdx.x * kDxCols;
    const int c = cb + 4 * lane;
    const int s = blockIdx.y;
    const int tb = s * tps, te = min(T, tb + tps);
    for (int e0 = 0; e0 < E; e0 += kDwExperts) {
        const int ne = min(kDwExperts, E - e0);
        float acc[kDwExperts][4];
#pragma unroll
        for (int e = 0; e < kDwExperts; ++e)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[e][q] = 0.f;
        if (c < H) {
            // 8 of the wave's tokens per iteration, all loads first (bytes in
            // flight); tokens past the split's end load row tb with weight 0
            for (int t = tb + wave; t < te; t += 32) {
                u32x2 xv[8];
                float gw[8][kDwExperts];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int tu = t + 4 * u;
                    const bool ok = tu < te;
                    xv[u] = *(const u32x2*)(x + (int64_t)(ok ? tu : tb) * H + c);
                    const float* g = G + (int64_t)(ok ? tu : tb) * E + e0;
#pragma unroll
                    for (int e = 0; e < kDwExperts; ++e) gw[u][e] = (ok && e < ne) ? g[e] : 0.f;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float xf[4] = {lo_bf16(xv[u][0]), hi_bf16(xv[u][0]), lo_bf16(xv[u][1]),
                                         hi_bf16(xv[u][1])};
#pragma unroll
                    for (int e = 0; e < kDwExperts; ++e)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            acc[e][q] = __builtin_fmaf(gw[u][e], xf[q], acc[e][q]);
                }
            }
        }
#pragma unroll
        for (int e = 0; e < kDwExperts; ++e)
#pragma unroll
            for (int q = 0; q < 4; ++q) red[wave][e][4 * lane + q] = acc[e][q];
        __syncthreads();
        for (int i = tid; i < ne * kDxCols; i += 256) {
            const int e = i / kDxCols, cl = i - e * kDxCols;
            if (cb + cl < H)
                part[((int64_t)s * E + e0 + e) * H + cb + cl] =
                    ((red[0][e][cl] + red[1][e][cl]) + red[2][e][cl]) + red[3][e][cl];
        }
        __syncthreads();
    }
}

// The same partial sums for more than kDwExperts experts, in one pass over x:
// lane l of every wave holds G[t][l] (expert l) of the wave's tokens and 2
// columns per lane for all 64 experts in registers; v_readlane hands each
// expert's weight to the whole wave.  The 4 waves are added in order, 16
// experts at a time through LDS.
constexpr int kDwCols64 = 128;      // columns per workgroup (2 per lane)
__global__ __launch_bounds__(256) void router_dw64_kernel(const float* __restrict__ G,
                                                          const bf16_t* __restrict__ x, int T,
                                                          int H, int E, int tps,
                                                          float* __restrict__ part) {
    __shared__ float red[4][16][kDwCols64 + 4];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane((int)(tid >> 6));
    const int lane = tid & 63;
    const int cb = blockIdx.x * kDwCols64;
    const int c = cb + 2 * lane;
    const int s = blockIdx.y;
    const int tb = s * tps, te = min(T, tb + tps);
    float acc[64][2];
#pragma unroll
    for (int e = 0; e < 64; ++e) acc[e][0] = acc[e][1] = 0.f;
    // Every lane stays active through the loop (v_readlane reads the lanes'
    // weights whatever the execution mask); lanes past the last column load
    // column 0 and use zeros.
    const bool col_ok = c < H;
    const int cl = col_ok ? c : 0;
    // 4 of the wave's tokens per iteration, loads first; tokens past the
    // split's end load row tb with weight 0
    for (int t = tb + wave; t < te; t += 16) {
        uint32_t xv[4];
        float gv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int tu = t + 4 * u;
            const bool ok = tu < te;
            const uint32_t xl = *(const uint32_t*)(x + (int64_t)(ok ? tu : tb) * H + cl);
            xv[u] = col_ok ? xl : 0u;
            const float gl = G[(int64_t)(ok ? tu : tb) * E + (lane < E ? lane : 0)];
            gv[u] = (ok && lane < E) ? gl : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float x0 = lo_bf16(xv[u]), x1 = hi_bf16(xv[u]);
#pragma unroll
            for (int e = 0; e < 64; ++e) {
                const float g = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gv[u]), e));
                acc[e][0] = __builtin_fmaf(g, x0, acc[e][0]);
                acc[e][1] = __builtin_fmaf(g, x1, acc[e][1]);
            }
        }
    }
#pragma unroll
    for (int e0 = 0; e0 < 64; e0 += 16) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            red[wave][e][2 * lane] = acc[e0 + e][0];
            red[wave][e][2 * lane + 1] = acc[e0 + e][1];
        }
        __syncthreads();
        for (int i = tid; i < 16 * kDwCols64; i += 256) {
            const int e = i / kDwCols64, cl = i - e * kDwCols64;
            if (e0 + e < E && cb + cl < H)
                part[((int64_t)s * E + e0 + e) * H + cb + cl] =
                    ((red[0][e][cl] + red[1][e][cl]) + red[2][e][cl]) + red[3][e][cl];
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void router_dw_reduce_kernel(const float* __restrict__ part,
                                                               int ns, int64_t n,
                                                               bf16_t* __restrict__ dw) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * 256) {
        float a = 0.f;
        for (int s = 0; s < ns; ++s) a += part[(int64_t)s * n + i];
        dw[i] = (bf16_t)f32_to_bf16(a);
    }
}

// ---------------------------------------------------------------- launchers
// Columns per weight-gradient workgroup: the many-expert kernel keeps all 64
// experts in registers for 2 columns per lane.
static int router_dw_cols(int E) { return E > kDwExperts ? kDwCols64 : kDxCols; }

// Token splits of the weight gradient: enough workgroups to cover the chip
// (about 512), at least 64 tokens each.
static int router_dw_splits(int64_t T, int H, int E) {
    const int cols = router_dw_cols(E);
    const int64_t ctiles = (H + cols - 1) / cols;
    int64_t ns = (512 + ctiles - 1) / ctiles;
    const int64_t cap = (T + 63) / 64;
    if (ns > cap) ns = cap;
    return (int)(ns < 1 ? 1 : ns);
}

size_t router_bwd_workspace_bytes(int64_t T, int H, int E) {
    return (size_t)router_dw_splits(T, H, E) * E * H * sizeof(float) + 256;
}

hipError_t launch_router_logits(const bf16_t* x, const bf16_t* w, int T, int H, int E,
                                float* logits, hipStream_t s) {
    if (T == 0) return hipSuccess;
    TraceScope ts("router_logits", s);
    router_logits_kernel<<<(T + kRtTok - 1) / kRtTok, 64 * kRtWaves, 0, s>>>(x, w, T, H, E,
                                                                            logits);
    return hipGetLastError();
}

hipError_t launch_router_bwd(const float* dlogits, const bf16_t* x, const bf16_t* w, int T,
                             int H, int E, int k, const int32_t* dest_row, const bf16_t* dxp,
                             bf16_t* dx, bf16_t* dw, void* ws, hipStream_t s) {
    if (T == 0) {
        // no tokens: dW_r = 0
        TraceScope ts("router_dw_reduce", s);
        const int64_t n = (int64_t)E * H;
        router_dw_reduce_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
            (const float*)ws, 0, n, dw);
        return hipGetLastError();
    }
    {
        TraceScope ts("router_dx", s);
        dim3 grid((unsigned)((H + kDxCols - 1) / kDxCols), (unsigned)((T + kDxTok - 1) / kDxTok));
        router_dx_kernel<<<grid, 256, 0, s>>>(dlogits, w, dxp, dest_row, T, H, E, k, dx);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int ns = router_dw_splits(T, H, E);
    const int tps = (T + ns - 1) / ns;
    float* part = (float*)ws;
    {
        TraceScope ts("router_dw", s);
        const int cols = router_dw_cols(E);
        dim3 grid((unsigned)((H + cols - 1) / cols), (unsigned)ns);
        if (E > kDwExperts)
            router_dw64_kernel<<<grid, 256, 0, s>>>(dlogits, x, T, H, E, tps, part);
        else
            router_dw_kernel<<<grid, 256, 0, s>>>(dlogits, x, T, H, E, tps, part);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    TraceScope ts("router_dw_reduce", s);
    const int64_t n = (int64_t)E * H;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    router_dw_reduce_kernel<<<(unsigned)blocks, 256, 0, s>>>(part, ns, n, dw);
    return hipGetLastError();
}

}  // namespace moe
