// MXFP8 block quantization and dequantization kernels for gfx950.
//
// One scale per 32 consecutive values, applied to BF16 weights and
// activations before the low-precision GEMMs and removed afterwards [BioNeMo
// MoE recipe page, bottleneck section and the section on MXFP8 and the fused
// MLP].  Encoding rules in common.hpp.
//
// Rowwise (blocks along the last dim): one thread per block of 32 values, 64 B
// read and 33 B written per thread.  Grouped columnwise (blocks of 32 rows
// inside each group, stored transposed so the rows become the contiguous
// axis): one thread per 4 columns of one 32-row block, so the block maximum
// is a per-thread reduction and each column's 32 codes leave as two 16 B
// stores.  Both are HBM-bound.
//
// The kernels take tables of matrices so that all experts' weights are
// quantized by one launch.
#include "common.hpp"
#include "kernels.hpp"
#include "trace.hpp"

namespace moe {

// ---------------------------------------------------------------- rowwise
__global__ __launch_bounds__(256) void quant_rows_kernel(MatTable src, MatTable codes,
                                                         MatTable scales, int nmat, int64_t rows,
                                                         int64_t cols, int scales_t) {
    const int64_t bpr = cols / kMxBlock;
    const int64_t per_mat = rows * bpr;
    const int64_t total = per_mat * nmat;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        int m = (int)(i / per_mat);
        int64_t b = i - (int64_t)m * per_mat;          // block index inside the matrix
        const u32x4* in = (const u32x4*)src.p[m] + b * 4;
        u32x4 v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = __builtin_nontemporal_load(in + q);
        float amax = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int w = 0; w < 4; ++w)
                amax = fmaxf(amax, fmaxf(__builtin_fabsf(lo_bf16(v[q][w])),
                                         __builtin_fabsf(hi_bf16(v[q][w]))));
        uint32_t S = mx_scale_byte(amax);
        u32x4 o[2];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            o[q >> 1][(q & 1) * 2] = mx_encode4(lo_bf16(v[q][0]), hi_bf16(v[q][0]),
                                                lo_bf16(v[q][1]), hi_bf16(v[q][1]), S);
            o[q >> 1][(q & 1) * 2 + 1] = mx_encode4(lo_bf16(v[q][2]), hi_bf16(v[q][2]),
                                                    lo_bf16(v[q][3]), hi_bf16(v[q][3]), S);
        }
        u32x4* out = (u32x4*)codes.p[m] + b * 2;
        out[0] = o[0];
        out[1] = o[1];
        int64_t si = b;
        if (scales_t) {                               // block-major: [cols/32][rows]
            int64_t r = b / bpr, kb = b - r * bpr;
            si = kb * rows + r;
        }
        ((uint8_t*)scales.p[m])[si] = (uint8_t)S;
    }
}

__global__ __launch_bounds__(256) void dequant_rows_kernel(const u32x4* __restrict__ codes,
                                                           const uint8_t* __restrict__ scales,
                                                           int64_t nblocks,
                                                           u32x4* __restrict__ out) {
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblocks;
         b += (int64_t)gridDim.x * blockDim.x) {
        u32x4 c[2] = {codes[2 * b], codes[2 * b + 1]};
        uint32_t S = scales[b];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t w0 = c[q >> 1][(q & 1) * 2], w1 = c[q >> 1][(q & 1) * 2 + 1];
            u32x4 o;
            o[0] = pack_bf16x2(mx_decode(w0 & 0xff, S), mx_decode((w0 >> 8) & 0xff, S));
            o[1] = pack_bf16x2(mx_decode((w0 >> 16) & 0xff, S), mx_decode(w0 >> 24, S));
            o[2] = pack_bf16x2(mx_decode(w1 & 0xff, S), mx_decode((w1 >> 8) & 0xff, S));
            o[3] = pack_bf16x2(mx_decode((w1 >> 16) & 0xff, S), mx_decode(w1 >> 24, S));
            out[4 * b + q] = o;
        }
    }
}

// ---------------------------------------------------------------- grouped columnwise
// Locates the 32-row block `q` (counted over all groups) of a grouped layout.
// Needs one full wave (lanes 0..63) of the calling block to be active.
struct ColBlock {
    int64_t r0;        // first input row of the block
    int valid;         // rows of the block that exist (1..32), 0 = past the end
    int64_t pad_rows;  // P_g of the block's group
    int64_t pbase;     // P_0 + .. + P_{g-1}
    int64_t i0;        // row of the block inside its (padded) group
};

__device__ ColBlock locate_col_block(const int32_t* __restrict__ sizes, int ngroups,
                                     int64_t rows, int64_t q, int* lds) {
    // lds: 3 * 64 ints; filled by the first wave.
    const int tid = threadIdx.x;
    if (tid < 64) {
        int n = 0;
        if (sizes) n = tid < ngroups ? sizes[tid] : 0;
        else n = tid == 0 ? (int)rows : 0;
        int nb = (n + kMxBlock - 1) / kMxBlock;
        int inb = wave_incl_scan(nb);
        int inr = wave_incl_scan(n);
        lds[tid] = inb;          // inclusive block prefix
        lds[64 + tid] = inr;     // inclusive row prefix
        lds[128 + tid] = n;
    }
    __syncthreads();
    ColBlock cb{0, 0, 0, 0, 0};
    int G = sizes ? ngroups : 1;
    int g = 0;
    while (g < G && lds[g] <= q) ++g;   // first group whose inclusive prefix passes q
    if (g >= G) return cb;
    int bex = g ? lds[g - 1] : 0;
    int rex = g ? lds[64 + g - 1] : 0;
    int n = lds[128 + g];
    cb.i0 = (q - bex) * kMxBlock;
    cb.r0 = rex + cb.i0;
    cb.valid = (int)min((int64_t)kMxBlock, (int64_t)n - cb.i0);
    cb.pad_rows = (int64_t)((n + kMxBlock - 1) / kMxBlock) * kMxBlock;
    cb.pbase = (int64_t)bex * kMxBlock;
    return cb;
}

// 256 threads x 4 columns; grid (ceil(cols/1024), upper bound of 32-row
// blocks, nmat).
__global__ __launch_bounds__(256) void quant_cols_kernel(MatTable src, MatTable codes,
                                                         MatTable scales,
                                                         const int32_t* __restrict__ sizes,
                                                         int ngroups, int64_t rows,
                                                         int64_t cols, int scales_t) {
    __shared__ int lds[192];
    const int m = blockIdx.z;
    ColBlock cb = locate_col_block(sizes, ngroups, rows, blockIdx.y, lds);
    if (cb.valid <= 0) return;
    const int64_t c0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (c0 >= cols) return;
    const bf16_t* in = (const bf16_t*)src.p[m];
    u32x2 v[kMxBlock];
#pragma unroll
    for (int i = 0; i < kMxBlock; ++i) {
        v[i] = (u32x2){0u, 0u};
        if (i < cb.valid) v[i] = *(const u32x2*)(in + (cb.r0 + i) * cols + c0);
    }
    uint8_t* cout = (uint8_t*)codes.p[m] + cb.pbase * cols + cb.i0;
    // scale of (column c, block i0/32): [c][P/32] (public) or [P/32][c] (block-major)
    uint8_t* sout = (uint8_t*)scales.p[m] + cb.pbase / kMxBlock * cols +
                    (scales_t ? cb.i0 / kMxBlock * cols : cb.i0 / kMxBlock);
    const int64_t sstride = scales_t ? 1 : cb.pad_rows / kMxBlock;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < kMxBlock; ++i) {
            uint32_t w = v[i][j >> 1];
            float f = (j & 1) ? hi_bf16(w) : lo_bf16(w);
            amax = fmaxf(amax, __builtin_fabsf(f));
        }
        uint32_t S = mx_scale_byte(amax);
        u32x4 o[2];
#pragma unroll
        for (int i = 0; i < kMxBlock; i += 4) {
            float f[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uint32_t w = v[i + r][j >> 1];
                f[r] = (j & 1) ? hi_bf16(w) : lo_bf16(w);
            }
            o[i >> 4][(i >> 2) & 3] = mx_encode4(f[0], f[1], f[2], f[3], S);
        }
        u32x4* dst = (u32x4*)(cout + (c0 + j) * cb.pad_rows);
        dst[0] = o[0];
        dst[1] = o[1];
        sout[(c0 + j) * sstride] = (uint8_t)S;
    }
}

__global__ __launch_bounds__(256) void dequant_cols_kernel(const uint8_t* __restrict__ codes,
                                                           const uint8_t* __restrict__ scales,
                                                           const int32_t* __restrict__ sizes,
                                                           int ngroups, int64_t rows,
                                                           int64_t cols,
                                                           bf16_t* __restrict__ out) {
    __shared__ int lds[192];
    ColBlock cb = locate_col_block(sizes, ngroups, rows, blockIdx.y, lds);
    if (cb.valid <= 0) return;
    const int64_t c0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (c0 >= cols) return;
    const uint8_t* cin = codes + cb.pbase * cols + cb.i0;
    const uint8_t* sin = scales + cb.pbase / kMxBlock * cols + cb.i0 / kMxBlock;
    const int64_t sstride = cb.pad_rows / kMxBlock;
    u32x4 c[4][2];
    uint32_t S[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const u32x4* src = (const u32x4*)(cin + (c0 + j) * cb.pad_rows);
        c[j][0] = src[0];
        c[j][1] = src[1];
        S[j] = sin[(c0 + j) * sstride];
    }
#pragma unroll
    for (int i = 0; i < kMxBlock; ++i) {
        if (i < cb.valid) {
            float f[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t w = c[j][i >> 4][(i >> 2) & 3];
                f[j] = mx_decode((w >> (8 * (i & 3))) & 0xff, S[j]);
            }
            *(u32x2*)(out + (cb.r0 + i) * cols + c0) =
                (u32x2){pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3])};
        }
    }
}

// ---------------------------------------------------------------- launchers
static unsigned grid_1d(int64_t n, int threads) {
    int64_t b = (n + threads - 1) / threads;
    int64_t cap = 256 * 32;
    return (unsigned)(b < 1 ? 1 : (b < cap ? b : cap));
}

int64_t colwise_block_bound(int64_t rows, int ngroups) {
    return (rows + kMxBlock - 1) / kMxBlock + (ngroups > 1 ? ngroups : 1);
}

hipError_t launch_quant_rows(const MatTable& src, const MatTable& codes, const MatTable& scales,
                             int nmat, int64_t rows, int64_t cols, hipStream_t s,
                             const char* name, bool scales_t) {
    int64_t n = (int64_t)nmat * rows * (cols / kMxBlock);
    if (n == 0) return hipSuccess;
    TraceScope ts(name, s);
    quant_rows_kernel<<<grid_1d(n, 256), 256, 0, s>>>(src, codes, scales, nmat, rows, cols,
                                                      scales_t ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_quant_cols(const MatTable& src, const MatTable& codes, const MatTable& scales,
                             int nmat, const int32_t* sizes, int ngroups, int64_t rows,
                             int64_t cols, hipStream_t s, const char* name, bool scales_t) {
    if (rows == 0 || cols == 0 || nmat == 0) return hipSuccess;
    dim3 grid((unsigned)((cols + 1023) / 1024), (unsigned)colwise_block_bound(rows, ngroups),
              (unsigned)nmat);
    TraceScope ts(name, s);
    quant_cols_kernel<<<grid, 256, 0, s>>>(src, codes, scales, sizes, ngroups, rows, cols,
                                           scales_t ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_dequant_rows(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                               int64_t cols, bf16_t* out, hipStream_t s) {
    int64_t nb = rows * (cols / kMxBlock);
    if (nb == 0) return hipSuccess;
    TraceScope ts("mx_dequant_rows", s);
    dequant_rows_kernel<<<grid_1d(nb, 256), 256, 0, s>>>((const u32x4*)codes, scales, nb,
                                                         (u32x4*)out);
    return hipGetLastError();
}

hipError_t launch_dequant_cols(const uint8_t* codes, const uint8_t* scales, const int32_t* sizes,
                               int ngroups, int64_t rows, int64_t cols, bf16_t* out,
                               hipStream_t s) {
    if (rows == 0 || cols == 0) return hipSuccess;
    dim3 grid((unsigned)((cols + 1023) / 1024), (unsigned)colwise_block_bound(rows, ngroups), 1);
    TraceScope ts("mx_dequant_cols", s);
    dequant_cols_kernel<<<grid, 256, 0, s>>>(codes, scales, sizes, ngroups, rows, cols, out);
    return hipGetLastError();
}

}  // namespace moe
