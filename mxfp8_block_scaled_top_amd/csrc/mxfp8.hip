// MXFP8 block quantization and dequantization kernels for gfx950.
//
// One scale per 32 consecutive values, applied to BF16 weights and
// activations before the low-precision GEMMs and removed afterwards [BioNeMo
// MoE recipe page, bottleneck section and the section on MXFP8 and the fused
// MLP].  Encoding rules in common.hpp.
//
// Quantization reads each value once and can write both orientations from
// that read: rowwise (blocks along the last dim) and grouped columnwise
// (blocks of 32 rows inside each group, stored transposed so the rows become
// the contiguous axis).  A weight needs both (forward and backward GEMMs
// contract it along different axes), and so do the activations that enter a
// data-gradient GEMM and a weight-gradient GEMM.  HBM-bound.
//
// The kernels take tables of matrices so that all experts' weights are
// quantized by one launch.
#include "common.hpp"
#include "kernels.hpp"
#include "trace.hpp"

namespace moe {

// ---------------------------------------------------------------- dequantization, rowwise
__global__ __launch_bounds__(256) void dequant_rows_kernel(const u32x4* __restrict__ codes,
                                                           const uint8_t* __restrict__ scales,
                                                           int64_t nblocks,
                                                           u32x4* __restrict__ out) {
    // A wave covers 64 consecutive 32-value blocks; in step q, lane l handles
    // 8 values: piece l&3 of block q*16 + l/4, so every load reads 512
    // contiguous code bytes and every store writes 1 KiB of whole lines.
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (nblocks + 63) / 64;
    const int64_t stride = (int64_t)gridDim.x * (blockDim.x / 64);
    const u32x2* cw = (const u32x2*)codes;
    for (int64_t w = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6); w < nwaves;
         w += stride) {
        u32x2 c[4];
        uint32_t S[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t blk = w * 64 + q * 16 + (lane >> 2);
            c[q] = (u32x2){0u, 0u};
            S[q] = 127u;
            if (blk < nblocks) {
                c[q] = cw[blk * 4 + (lane & 3)];
                S[q] = scales[blk];
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t blk = w * 64 + q * 16 + (lane >> 2);
            if (blk < nblocks) {
                // gfx950's scaled conversion, two codes per instruction: each
                // code times 2^(S-127), rounded to nearest even bf16 (the same
                // bits as mx_decode followed by that rounding, for every code
                // and scale byte, overflow to infinity and underflow included)
                const float scale = __builtin_ldexpf(1.f, (int)S[q] - 127);
                u32x4 o;
                o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[q][0], scale, false));
                o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[q][0], scale, true));
                o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[q][1], scale, false));
                o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[q][1], scale, true));
                out[blk * 4 + (lane & 3)] = o;
            }
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
    int64_t pad64;     // the group's size padded to 64, and the sum of those of
    int64_t pbase64;   // the earlier groups (row-pair grouped layout)
};

__device__ ColBlock locate_col_block(const int32_t* __restrict__ sizes, int ngroups,
                                     int64_t rows, int64_t q, int* lds) {
    // lds: 4 * 64 ints; filled by the first wave.
    const int tid = threadIdx.x;
    if (tid < 64) {
        int n = 0;
        if (sizes) n = tid < ngroups ? sizes[tid] : 0;
        else n = tid == 0 ? (int)rows : 0;
        n = clamp_group_size(n, rows);
        int nb = (n + kMxBlock - 1) / kMxBlock;
        int inb = wave_incl_scan(nb);
        int inr = wave_incl_scan(n);
        lds[tid] = inb;          // inclusive block prefix
        lds[64 + tid] = inr;     // inclusive row prefix
        lds[128 + tid] = n;
        lds[192 + tid] = wave_incl_scan((n + 63) / 64);   // inclusive 64-row-chunk prefix
    }
    __syncthreads();
    ColBlock cb{0, 0, 0, 0, 0, 0, 0};
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
    cb.pad64 = (int64_t)((n + 63) / 64) * 64;
    cb.pbase64 = (int64_t)(g ? lds[192 + g - 1] : 0) * 64;
    return cb;
}

// ---------------------------------------------------------------- quantization
// One launch quantizes a bf16 matrix (or one per expert) rowwise, grouped
// columnwise, or both from a single read of its values.
//
// A wave takes one 32-row block of the grouped walk (the blocks of the
// columnwise layout; one group of all rows when there are no groups) and 512
// columns: lane l loads columns c0 = 512 * blockIdx.x + 8 l .. c0 + 7 of every
// row of the block, one 16-byte load per row (1 KiB per wave and row).
//   rowwise     a 32-value block is 4 neighbouring lanes; their maxima meet by
//               a quad reduction (DPP), and each lane encodes its 8 values and
//               stores them as 8 bytes (512 contiguous bytes per wave and row).
//   columnwise  a lane owns 8 whole 32-row column blocks: the maximum is a
//               per-lane reduction.  Block q of the walk goes to wave q % 4 of
//               workgroup q / 4, so the four waves of a workgroup hold the
//               four neighbouring 32-byte pieces of each column's 128 codes.
//               When the four blocks share a group and all 512 columns
//               exist, the codes meet in LDS and leave as 128-byte runs,
//               eight threads to a column (whole lines when the group's
//               padded size and start are multiples of 128); otherwise
//               two neighbouring lanes store each column's 32 codes as one
//               32-byte run.
// Block maxima are taken on the bf16 bit patterns with the sign cleared
// (ordered like the magnitudes), two at a time with packed 16-bit maxima.
struct QuantTileArgs {
    MatTable src;               // bf16 [rows, cols] per matrix
    MatTable rcodes, rscales;   // rowwise codes [rows, cols]; scales [rows][cols/32]
                                // or block-major [cols/32][rows]
    MatTable ccodes, cscales;   // grouped columnwise codes; scales [cols][P_g/32] or
                                // block-major [P_g/32][cols] per group
    const int32_t* sizes;       // group sizes (device), NULL = one group
    int ngroups;
    int64_t rows, cols;
    int rscales_t, cscales_t;
    int p2;                     // GEMM operand layouts: row codes in the row-pair
                                // layout at expert-padded rows (scales [cols/32]
                                // [rows_pad]); grouped columnwise codes in the
                                // row-pair layout of each group's 64-padded rows
    int64_t rows_pad;
    const float* amax;          // per-tensor mode: amax of matrix m (one scale for all
                                // its blocks, still written to every scale slot)
    const int32_t* gather;      // one matrix: row r is read from source row gather[r]
};

typedef __attribute__((ext_vector_type(2))) unsigned short u16x2;

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

// magnitude bits of the two bf16 halves of w
__device__ __forceinline__ uint32_t abs2(uint32_t w) { return w & 0x7fff7fffu; }

template <bool ROWS, bool COLS, bool FIXED, bool GATHER>
__global__ __launch_bounds__(256) void quant_tile_kernel(QuantTileArgs a) {
    __shared__ int lds[256];
    const int m = blockIdx.z;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    const ColBlock cb = locate_col_block(a.sizes, a.ngroups, a.rows,
                                         (int64_t)blockIdx.y * 4 + wv, lds);
    // The workgroup's four blocks lie in one group and its 512 columns all
    // exist: its column codes then leave through LDS as whole 128-byte lines
    // (the four blocks' 32-byte pieces of a column are neighbours).
    bool staged = false;
    if constexpr (COLS) {
        const int G = a.sizes ? a.ngroups : 1;
        const int q0 = (int)blockIdx.y * 4;
        int g0 = 0, g3 = 0;
        while (g0 < G && lds[g0] <= q0) ++g0;
        while (g3 < G && lds[g3] <= q0 + 3) ++g3;
        staged = g3 < G && g0 == g3 && (int64_t)(blockIdx.x + 1) * 512 <= a.cols;
    }
    // every field is the same across the wave
    const int valid = __builtin_amdgcn_readfirstlane(cb.valid);
    if (valid <= 0) return;
    const int64_t r0 = __builtin_amdgcn_readfirstlane((int)cb.r0);
    const int64_t i0 = __builtin_amdgcn_readfirstlane((int)cb.i0);
    const int64_t pad = __builtin_amdgcn_readfirstlane((int)cb.pad_rows);
    const int64_t pbase = __builtin_amdgcn_readfirstlane((int)cb.pbase);
    const int64_t pad64 = __builtin_amdgcn_readfirstlane((int)cb.pad64);
    const int64_t pbase64 = __builtin_amdgcn_readfirstlane((int)cb.pbase64);
    const int64_t cols = a.cols;
    const int64_t c0 = (int64_t)blockIdx.x * 512 + lane * 8;
    // lanes stay in pairs (the columnwise stores need both); rowwise, cols is
    // a multiple of 32, so both lanes of a pair always hold columns
    if ((c0 & ~(int64_t)15) >= cols) return;
    const bool live = c0 < cols;

    u32x4 v[kMxBlock];
    if constexpr (GATHER) {
        // row r0 + j of the block is source row gather[r0 + j] (the same for
        // the whole wave: scalar loads).  Ordinary loads, not streaming ones:
        // each token row is read k times, and with many experts and k = 8
        // some of the other reads find it still in L2 (E = 64, k = 8: 0.225
        // -> 0.21 ms per launch; no change at E = 8, k = 2).
        const char* in = (const char*)a.src.p[m] + c0 * 2;
        int64_t srow[kMxBlock];
#pragma unroll
        for (int j = 0; j < kMxBlock; ++j) srow[j] = j < valid ? a.gather[r0 + j] : 0;
#pragma unroll
        for (int j = 0; j < kMxBlock; ++j) {
            v[j] = (u32x4){0u, 0u, 0u, 0u};
            if (j < valid && live) v[j] = *(const u32x4*)(in + srow[j] * cols * 2);
        }
    } else {
        const char* in = (const char*)a.src.p[m] + r0 * cols * 2;
#pragma unroll
        for (int j = 0; j < kMxBlock; ++j) {
            v[j] = (u32x4){0u, 0u, 0u, 0u};
            if (j < valid && live)
                v[j] = __builtin_nontemporal_load((const u32x4*)(in + (j * cols + c0) * 2));
        }
    }

    uint32_t Sfix = 0;
    if constexpr (FIXED) Sfix = mx_scale_byte(a.amax[m]);

    if constexpr (ROWS) {
        // public layout: row r0 + j at (r0 + j) * cols; row-pair layout: row
        // pbase + i0 + j (its expert-padded position), 8 bytes per lane
        // within one 64-byte half line
        const int64_t ps = p2_stride(cols);
        const int64_t rq = pbase + i0;
        uint8_t* rc = (uint8_t*)a.rcodes.p[m] + r0 * cols + c0;
        uint8_t* rcp = (uint8_t*)a.rcodes.p[m] + (rq >> 1) * ps + (c0 >> 6) * 128 + (c0 & 63);
        const int64_t kb = c0 >> 5;
        const int s = lane & 3;
        uint32_t sp[2] = {0u, 0u};   // block-major: scale bytes of rows 8s .. 8s+7
#pragma unroll
        for (int j = 0; j < kMxBlock; ++j) {
            if (j < valid) {
                uint32_t S = Sfix;
                if constexpr (!FIXED) {
                    uint32_t mw = pk_max_u16(pk_max_u16(abs2(v[j][0]), abs2(v[j][1])),
                                             pk_max_u16(abs2(v[j][2]), abs2(v[j][3])));
                    uint32_t am = max(mw & 0xffffu, mw >> 16);
                    // quad_perm [1,0,3,2] then [2,3,0,1]: the 4 lanes of a block
                    am = max(am, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)am, 0xB1, 0xF, 0xF, true));
                    am = max(am, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)am, 0x4E, 0xF, 0xF, true));
                    S = mx_scale_byte(__uint_as_float(am << 16));
                }
                u32x2 o;
                o[0] = mx_encode4(lo_bf16(v[j][0]), hi_bf16(v[j][0]), lo_bf16(v[j][1]),
                                  hi_bf16(v[j][1]), S);
                o[1] = mx_encode4(lo_bf16(v[j][2]), hi_bf16(v[j][2]), lo_bf16(v[j][3]),
                                  hi_bf16(v[j][3]), S);
                if (a.p2) {   // rq is even: row j is half j & 1 of pair (rq + j) / 2
                    *(u32x2*)(rcp + (j >> 1) * ps + (j & 1) * 64) = o;
                } else {      // whole 512-byte runs per instruction: streamed past L2
                    __builtin_nontemporal_store(o, (u32x2*)(rc + j * cols));
                }
                if (a.rscales_t) {
                    if ((j >> 3) == s) sp[(j >> 2) & 1] |= S << (8 * (j & 3));
                } else if (s == 0) {
                    ((uint8_t*)a.rscales.p[m])[(r0 + j) * (cols >> 5) + kb] = (uint8_t)S;
                }
            }
        }
        if (a.rscales_t) {
            // [cols/32][rows]: this block's 32 rows of column block kb are
            // contiguous; lane s of the quad stores rows 8s .. 8s+7
            uint8_t* rs = (uint8_t*)a.rscales.p[m] +
                          (a.p2 ? kb * a.rows_pad + rq : kb * a.rows + r0) + 8 * s;
            const int nv = min(8, valid - 8 * s);
            if (nv == 8 && ((uintptr_t)rs & 7u) == 0) {
                *(u32x2*)rs = (u32x2){sp[0], sp[1]};
            } else {
                for (int t = 0; t < nv; ++t) rs[t] = (uint8_t)(sp[t >> 2] >> (8 * (t & 3)));
            }
        }
    }

    if constexpr (ROWS && COLS) {
        // keeps the compiler from holding the rowwise pass's 256 widened
        // floats live for reuse here (that would cost the occupancy)
#pragma unroll
        for (int j = 0; j < kMxBlock; ++j) asm volatile("" : "+v"(v[j]));
    }

    if constexpr (COLS) {
        uint32_t mw[4] = {0u, 0u, 0u, 0u};   // column maxima, two columns per word
#pragma unroll
        for (int j = 0; j < kMxBlock; ++j)
#pragma unroll
            for (int w = 0; w < 4; ++w) mw[w] = pk_max_u16(mw[w], abs2(v[j][w]));
        // group g stored as [cols, P_g] at cols * P_0..g-1 (public layout) or
        // in the row-pair layout of [cols, 64-padded rows] at cols * the sum
        // of the earlier groups' 64-padded sizes; rows past the group's end
        // were loaded as zeros and encode to 0x00.  colrun(c, i) is where
        // column c's codes of group rows i .. i + 31 start (32 contiguous bytes).
        uint8_t* cc = (uint8_t*)a.ccodes.p[m] + pbase * cols + i0;
        uint8_t* ccp = (uint8_t*)a.ccodes.p[m] + pbase64 * cols;
        const int64_t cps = 2 * pad64;
        auto colrun = [&](int64_t c, int64_t i) -> uint8_t* {
            return a.p2 ? ccp + p2_off(c, i, cps) : cc + c * pad + (i - i0);
        };
        // staged: 256 column lines of 128 bytes (rows i0 - 32 wv .. + 127),
        // half the workgroup's columns at a time.  Line li (lane li / 4,
        // column t = li % 4 of the half) sits at slot li ^ bit 5 of li, its
        // 16-byte pieces rotated by lane % 8, so neither the writes nor the
        // reads meet on an LDS bank.
        __shared__ u32x4 stage[256 * 8];
        uint32_t sc[2] = {0u, 0u};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const int t = 4 * h + tt;
                const uint32_t am = (t & 1) ? (mw[t >> 1] >> 16) : (mw[t >> 1] & 0xffffu);
                const uint32_t S = FIXED ? Sfix : mx_scale_byte(__uint_as_float(am << 16));
                u32x4 o[2];
#pragma unroll
                for (int q = 0; q < 8; ++q) {   // rows 4q .. 4q+3
                    float f[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const uint32_t w = v[4 * q + r][t >> 1];
                        f[r] = (t & 1) ? hi_bf16(w) : lo_bf16(w);
                    }
                    o[q >> 2][q & 3] = mx_encode4(f[0], f[1], f[2], f[3], S);
                }
                sc[t >> 2] |= S << (8 * (t & 3));
                if (staged) {
                    const int li = 4 * lane + tt;
                    const int slot = li ^ ((li >> 5) & 1);
                    stage[slot * 8 + ((2 * wv) ^ (lane & 7))] = o[0];
                    stage[slot * 8 + ((2 * wv + 1) ^ (lane & 7))] = o[1];
                    continue;
                }
                // lanes 2p and 2p + 1 trade halves so that each store writes
                // the 32 codes of one column as 32 contiguous bytes over two
                // lanes: first the even lane's column, then the odd lane's
                const bool odd = lane & 1;
                const u32x4 send = odd ? o[0] : o[1];
                u32x4 recv;
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    recv[d] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send[d], 0xB1, 0xF, 0xF, true);
                const int64_t ce = (c0 & ~(int64_t)15) + t;   // the even lane's column
                *(u32x4*)(colrun(ce, i0) + (odd ? 16 : 0)) = odd ? recv : o[0];
                if ((c0 | 8) < cols)
                    *(u32x4*)(colrun(ce + 8, i0) + (odd ? 16 : 0)) = odd ? o[1] : recv;
            }
            if (staged) {
                __syncthreads();
                // eight neighbouring threads store one column's 128 codes
                // (piece p: rows i0b + 16p .. + 15): streamed past L2 when the
                // instruction fills whole lines, else plain stores (a run
                // across two lines shares each with another workgroup).  In
                // the row-pair layout the pieces of columns 2c and 2c+1 from
                // a 64-row boundary fill two lines.
                const int64_t i0b = i0 - 32 * wv;
                uint8_t* cw = cc - 32 * wv;
                const bool whole = a.p2 ? (i0b & 63) == 0
                                        : (pad & 127) == 0 && ((uintptr_t)cw & 127) == 0;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int ch = k * 256 + (int)threadIdx.x;
                    const int li = ch >> 3, piece = ch & 7;
                    const int slot = li ^ ((li >> 5) & 1);
                    const u32x4 val = stage[slot * 8 + (piece ^ ((li >> 2) & 7))];
                    const int64_t col = (int64_t)blockIdx.x * 512 + 8 * (li >> 2) + (li & 3) + 4 * h;
                    u32x4* dst = (u32x4*)(a.p2 ? ccp + p2_off(col, i0b + 16 * piece, cps)
                                               : cw + col * pad + 16 * piece);
                    if (whole) __builtin_nontemporal_store(val, dst);
                    else *dst = val;
                }
                __syncthreads();
            }
        }
        uint8_t* cs = (uint8_t*)a.cscales.p[m] + pbase / kMxBlock * cols;
        if (!live) {
        } else if (a.cscales_t) {   // [P_g/32][cols]: 8 neighbouring columns, 8 bytes
            *(u32x2*)(cs + i0 / kMxBlock * cols + c0) = (u32x2){sc[0], sc[1]};
        } else {             // [cols][P_g/32]
#pragma unroll
            for (int t = 0; t < 8; ++t)
                cs[(c0 + t) * (pad / kMxBlock) + i0 / kMxBlock] =
                    (uint8_t)(sc[t >> 2] >> (8 * (t & 3)));
        }
    }
}

// ---------------------------------------------------------------- rowwise, public layout
// Rowwise MXFP8 of one matrix into the public layout (codes [rows, cols],
// scales [rows][cols/32]), the standalone quantization.  A wave takes chunks
// of 4 rows x 512 columns (lane l: columns 8l .. 8l+7 of each row), chunk
// w, w + W, w + 2W, ... for wave w of W, and issues the loads of its next
// chunk before it encodes the current one, so that every wave keeps a chunk
// of loads in flight through its encoding and stores.  Block maxima as in
// quant_tile (bf16 magnitude bits, quad reduction over the 4 lanes of a
// 32-value block).
__device__ __forceinline__ void rows_chunk_load(const bf16_t* __restrict__ x, int64_t rows,
                                                int64_t cols, int64_t ncc, int64_t ch,
                                                int64_t nch, int lane, u32x4 (&v)[4]) {
    const int64_t rc = ch / ncc, cc = ch - rc * ncc;
    const int64_t r0 = rc * 4, c0 = cc * 512 + lane * 8;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[j] = (u32x4){0u, 0u, 0u, 0u};
        if (ch < nch && r0 + j < rows && c0 < cols)
            v[j] = __builtin_nontemporal_load((const u32x4*)(x + (r0 + j) * cols + c0));
    }
}

__device__ __forceinline__ void rows_chunk_encode(int64_t rows, int64_t cols, int64_t ncc,
                                                  int64_t ch, int lane, const u32x4 (&v)[4],
                                                  uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scales) {
    const int64_t rc = ch / ncc, cc = ch - rc * ncc;
    const int64_t r0 = rc * 4, c0 = cc * 512 + lane * 8;
    const bool live = c0 < cols;        // cols % 32 == 0: a quad is live or not as a whole
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t mw = pk_max_u16(pk_max_u16(abs2(v[j][0]), abs2(v[j][1])),
                                 pk_max_u16(abs2(v[j][2]), abs2(v[j][3])));
        uint32_t am = max(mw & 0xffffu, mw >> 16);
        am = max(am, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)am, 0xB1, 0xF, 0xF, true));
        am = max(am, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)am, 0x4E, 0xF, 0xF, true));
        const uint32_t S = mx_scale_byte(__uint_as_float(am << 16));
        if (r0 + j < rows && live) {
            u32x2 o;
            o[0] = mx_encode4(lo_bf16(v[j][0]), hi_bf16(v[j][0]), lo_bf16(v[j][1]),
                              hi_bf16(v[j][1]), S);
            o[1] = mx_encode4(lo_bf16(v[j][2]), hi_bf16(v[j][2]), lo_bf16(v[j][3]),
                              hi_bf16(v[j][3]), S);
            __builtin_nontemporal_store(o, (u32x2*)(codes + (r0 + j) * cols + c0));
            if ((lane & 3) == 0) scales[(r0 + j) * (cols >> 5) + (c0 >> 5)] = (uint8_t)S;
        }
    }
}

__global__ __launch_bounds__(256) void quant_rows_kernel(const bf16_t* __restrict__ x,
                                                         int64_t rows, int64_t cols,
                                                         uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales) {
    const int lane = threadIdx.x & 63;
    const int64_t W = (int64_t)gridDim.x * 4;
    const int64_t ncc = (cols + 511) / 512, nch = ncc * ((rows + 3) / 4);
    int64_t ch = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    u32x4 va[4], vb[4];
    rows_chunk_load(x, rows, cols, ncc, ch, nch, lane, va);
    // two register sets in turn (no copies): load the next chunk, encode this one
    while (ch < nch) {
        rows_chunk_load(x, rows, cols, ncc, ch + W, nch, lane, vb);
        rows_chunk_encode(rows, cols, ncc, ch, lane, va, codes, scales);
        ch += W;
        if (ch >= nch) break;
        rows_chunk_load(x, rows, cols, ncc, ch + W, nch, lane, va);
        rows_chunk_encode(rows, cols, ncc, ch, lane, vb, codes, scales);
        ch += W;
    }
}

__global__ __launch_bounds__(256) void dequant_cols_kernel(const uint8_t* __restrict__ codes,
                                                           const uint8_t* __restrict__ scales,
                                                           const int32_t* __restrict__ sizes,
                                                           int ngroups, int64_t rows,
                                                           int64_t cols,
                                                           bf16_t* __restrict__ out) {
    __shared__ int lds[256];
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

// ---------------------------------------------------------------- per-tensor amax
// Maximum magnitude of each of nmat bf16 matrices (n values each, n a
// multiple of 8), in two launches: workgroup partials over 16-byte chunks
// (magnitudes compared as bf16 bit patterns with the sign cleared), then one
// workgroup per matrix over its partials.  The maximum does not depend on
// the order, so the result is exact and deterministic.
constexpr int kAmaxParts = 512;

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    v = red[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) v = max(v, red[w]);
    return v;
}

__global__ __launch_bounds__(256) void amax_partial_kernel(MatTable src, int64_t n,
                                                           uint32_t* __restrict__ part) {
    __shared__ uint32_t red[4];
    const int m = blockIdx.y;
    const u32x4* p = (const u32x4*)src.p[m];
    uint32_t mw = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n / 8;
         i += (int64_t)gridDim.x * 256) {
        const u32x4 v = __builtin_nontemporal_load(p + i);
        mw = pk_max_u16(mw, pk_max_u16(pk_max_u16(abs2(v[0]), abs2(v[1])),
                                       pk_max_u16(abs2(v[2]), abs2(v[3]))));
    }
    const uint32_t am = block_max_u32(max(mw & 0xffffu, mw >> 16), red);
    if (threadIdx.x == 0) part[(int64_t)m * gridDim.x + blockIdx.x] = am;
}

// The same partials over the rows of a gathered matrix (row r of it is source
// row gather[r]): workgroup b takes rows b, b + gridDim.x, ...
__global__ __launch_bounds__(256) void amax_gather_partial_kernel(const u32x4* __restrict__ x,
                                                                  const int32_t* __restrict__ gather,
                                                                  int64_t rows, int64_t cpr,
                                                                  uint32_t* __restrict__ part) {
    __shared__ uint32_t red[4];
    uint32_t mw = 0;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const u32x4* p = x + (int64_t)gather[r] * cpr;
        for (int64_t c = threadIdx.x; c < cpr; c += 256) {
            const u32x4 v = __builtin_nontemporal_load(p + c);
            mw = pk_max_u16(mw, pk_max_u16(pk_max_u16(abs2(v[0]), abs2(v[1])),
                                           pk_max_u16(abs2(v[2]), abs2(v[3]))));
        }
    }
    const uint32_t am = block_max_u32(max(mw & 0xffffu, mw >> 16), red);
    if (threadIdx.x == 0) part[blockIdx.x] = am;
}

__global__ __launch_bounds__(256) void amax_final_kernel(const uint32_t* __restrict__ part,
                                                         int nparts, float* __restrict__ amax) {
    __shared__ uint32_t red[4];
    const int m = blockIdx.x;
    uint32_t v = 0;
    for (int i = threadIdx.x; i < nparts; i += 256) v = max(v, part[(int64_t)m * nparts + i]);
    v = block_max_u32(v, red);
    if (threadIdx.x == 0) amax[m] = __uint_as_float(v << 16);
}

// ---------------------------------------------------------------- launchers
hipError_t launch_amax_final(const uint32_t* part, int nparts, float* amax, hipStream_t s,
                             const char* name) {
    TraceScope ts(name, s);
    amax_final_kernel<<<1, 256, 0, s>>>(part, nparts, amax);
    return hipGetLastError();
}

size_t amax_workspace_bytes(int nmat) { return (size_t)nmat * kAmaxParts * sizeof(uint32_t) + 256; }

hipError_t launch_amax(const MatTable& src, int nmat, int64_t n, void* ws, float* amax,
                       hipStream_t s, const char* name) {
    if (nmat == 0) return hipSuccess;
    int64_t parts = (n / 8 + 255) / 256;
    if (parts > kAmaxParts) parts = kAmaxParts;
    if (parts < 1) parts = 1;
    TraceScope ts(name, s);
    amax_partial_kernel<<<dim3((unsigned)parts, (unsigned)nmat), 256, 0, s>>>(src, n,
                                                                            (uint32_t*)ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    amax_final_kernel<<<nmat, 256, 0, s>>>((const uint32_t*)ws, (int)parts, amax);
    return hipGetLastError();
}

hipError_t launch_amax_gather(const bf16_t* x, const int32_t* gather, int64_t rows, int64_t cols,
                              void* ws, float* amax, hipStream_t s, const char* name) {
    int64_t parts = rows < kAmaxParts ? rows : kAmaxParts;
    if (parts < 1) parts = 1;
    TraceScope ts(name, s);
    amax_gather_partial_kernel<<<(unsigned)parts, 256, 0, s>>>((const u32x4*)x, gather, rows,
                                                              cols / 8, (uint32_t*)ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    amax_final_kernel<<<1, 256, 0, s>>>((const uint32_t*)ws, (int)parts, amax);
    return hipGetLastError();
}

static unsigned grid_1d(int64_t n, int threads) {
    int64_t b = (n + threads - 1) / threads;
    int64_t cap = 256 * 32;
    return (unsigned)(b < 1 ? 1 : (b < cap ? b : cap));
}

int64_t colwise_block_bound(int64_t rows, int ngroups) {
    return (rows + kMxBlock - 1) / kMxBlock + (ngroups > 1 ? ngroups : 1);
}

// Quantizes nmat matrices of [rows, cols]: rowwise where rcodes is given,
// grouped columnwise where ccodes is given, both from one read.
hipError_t launch_quant(const MatTable& src, int nmat, const int32_t* sizes, int ngroups,
                        int64_t rows, int64_t cols, const MatTable* rcodes,
                        const MatTable* rscales, bool rscales_t, const MatTable* ccodes,
                        const MatTable* cscales, bool cscales_t, hipStream_t s,
                        const char* name, const float* fixed_amax, int64_t p2_rows_pad,
                        const int32_t* gather) {
    if (rows == 0 || cols == 0 || nmat == 0 || (!rcodes && !ccodes)) return hipSuccess;
    if (gather && nmat != 1) return hipErrorInvalidValue;
    QuantTileArgs a{};
    a.src = src;
    a.gather = gather;
    if (rcodes) a.rcodes = *rcodes, a.rscales = *rscales;
    if (ccodes) a.ccodes = *ccodes, a.cscales = *cscales;
    a.sizes = sizes;
    a.ngroups = sizes ? ngroups : 1;
    a.rows = rows;
    a.cols = cols;
    a.rscales_t = rscales_t ? 1 : 0;
    a.cscales_t = cscales_t ? 1 : 0;
    a.amax = fixed_amax;
    a.p2 = p2_rows_pad > 0 ? 1 : 0;
    a.rows_pad = p2_rows_pad;
    const int64_t nblk = colwise_block_bound(rows, a.ngroups);
    dim3 grid((unsigned)((cols + 511) / 512), (unsigned)((nblk + 3) / 4), (unsigned)nmat);
    TraceScope ts(name, s);
    if (gather) {   // the routed activations: both orientations
        if (!rcodes || !ccodes) return hipErrorInvalidValue;
        if (fixed_amax) quant_tile_kernel<true, true, true, true><<<grid, 256, 0, s>>>(a);
        else quant_tile_kernel<true, true, false, true><<<grid, 256, 0, s>>>(a);
    } else if (fixed_amax) {
        if (rcodes && ccodes) quant_tile_kernel<true, true, true, false><<<grid, 256, 0, s>>>(a);
        else if (rcodes) quant_tile_kernel<true, false, true, false><<<grid, 256, 0, s>>>(a);
        else quant_tile_kernel<false, true, true, false><<<grid, 256, 0, s>>>(a);
    } else {
        if (rcodes && ccodes) quant_tile_kernel<true, true, false, false><<<grid, 256, 0, s>>>(a);
        else if (rcodes) quant_tile_kernel<true, false, false, false><<<grid, 256, 0, s>>>(a);
        else quant_tile_kernel<false, true, false, false><<<grid, 256, 0, s>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_quant_rows(const MatTable& src, const MatTable& codes, const MatTable& scales,
                             int nmat, int64_t rows, int64_t cols, hipStream_t s,
                             const char* name, bool scales_t, int64_t p2_rows_pad) {
    if (nmat == 1 && !scales_t && p2_rows_pad == 0) {   // one matrix, public layout
        if (rows == 0 || cols == 0) return hipSuccess;
        // one chunk per wave up to 32768 waves (the most parallel loads: 20.2-21.2
        // us against 21.3-21.7 with 8-row chunks and 23-24 with 16-row ones on
        // 8192 x 4096); larger matrices loop with their next chunk's loads ahead
        const int64_t nch = ((cols + 511) / 512) * ((rows + 3) / 4);
        int64_t wg = (nch + 3) / 4;
        wg = wg < 1 ? 1 : (wg > 8192 ? 8192 : wg);
        TraceScope ts(name, s);
        quant_rows_kernel<<<(unsigned)wg, 256, 0, s>>>((const bf16_t*)src.p[0], rows, cols,
                                                      (uint8_t*)codes.p[0],
                                                      (uint8_t*)scales.p[0]);
        return hipGetLastError();
    }
    return launch_quant(src, nmat, nullptr, 1, rows, cols, &codes, &scales, scales_t, nullptr,
                        nullptr, false, s, name, nullptr, p2_rows_pad);
}

hipError_t launch_quant_cols(const MatTable& src, const MatTable& codes, const MatTable& scales,
                             int nmat, const int32_t* sizes, int ngroups, int64_t rows,
                             int64_t cols, hipStream_t s, const char* name, bool scales_t,
                             int64_t p2_rows_pad) {
    return launch_quant(src, nmat, sizes, ngroups, rows, cols, nullptr, nullptr, false, &codes,
                        &scales, scales_t, s, name, nullptr, p2_rows_pad);
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
