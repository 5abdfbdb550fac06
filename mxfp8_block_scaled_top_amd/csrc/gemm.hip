// Grouped GEMM over all experts in one launch, for gfx950 (CDNA4).
//
// The grouped call replaces one GEMM launch per expert [BioNeMo MoE recipe
// page, section GroupedLinear: all local experts' linear maps in one call,
// each expert with its own weight and its own number of rows]; SwiGLU, the
// routing-probability scale and the MXFP8 requantization are done in the
// GEMM epilogue so no intermediate goes to memory in a wider format than the
// next GEMM reads [same page, section on MXFP8 and the fused MLP].
//
// Work decomposition
//   * 256 x 256 output tile per workgroup of 512 threads (8 waves, 2 x 4);
//     every wave owns a 128 x 64 sub-tile = 4 x 2 MFMA 32x32 fragments.
//   * K steps of 128 bytes per operand row: 64 bf16 (4 x
//     v_mfma_f32_32x32x16_bf16) or 128 E4M3 (2 x
//     v_mfma_scale_f32_32x32x64_f8f6f4 with one E8M0 scale per 32 K-values
//     and row, fed straight to the instruction).
//   * Operand tiles are staged through LDS, double-buffered (2 x 64 KiB):
//     the next K step is loaded to registers while the current one feeds the
//     MFMAs.  16-byte chunks of a 128-byte LDS row are XOR-swizzled by
//     (row ^ row >> 3) & 7 so the 16-byte fragment reads of 16 consecutive
//     rows hit distinct banks.
//   * Operands contiguous along M/N (the bf16 weight-gradient and dgrad
//     operands) are loaded as 4 K-rows x 8 elements per thread and transposed
//     in registers before the LDS store, so every LDS row is K-contiguous.
//   * Grouping: the tile list is the concatenation over experts of their
//     tiles (ragged M: ceil(M_e / 256) x N-tiles each; ragged K: a fixed
//     M x N grid each, looping over the expert's rows).  The per-expert prefix
//     sums are rebuilt on the device from split_sizes by the first wave of
//     every workgroup.  Workgroup ids are remapped so that each of the 8 XCDs
//     (round-robin dispatch) gets a contiguous run of tiles: the M tiles that
//     share a weight tile run on the same XCD and share its L2.
//   * No float atomics: the probability gradient is written as per-(row,
//     N-tile) partial sums and reduced in a fixed order by a second kernel.
#include "common.hpp"
#include "kernels.hpp"
#include "mlp.hpp"
#include "trace.hpp"

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) int i32x8;

constexpr int kRowB = 128;                    // LDS bytes per tile row per K step
constexpr int kTileB = kGemmBM * kRowB;       // 32 KiB per operand per stage
constexpr int kStageB = 2 * kTileB;           // A + B
constexpr int kLdsB = 2 * kStageB;            // double-buffered: 128 KiB

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * kRowB + ((chunk ^ swz(row)) << 4);
}

// Per-workgroup tile descriptor.
struct Tile {
    int e;           // expert
    int m0, n0;      // first row (inside the expert for G_M) / column of the tile
    int64_t row0;    // first grouped row of the expert
    int rows_e;      // M_e (= K extent for G_K)
    int64_t pbase;   // sum of the padded (32) sizes of earlier experts
    int pad_e;       // padded size of this expert
    int n_tile;
};

// Builds the per-expert prefix tables in LDS and decodes the tile.  Returns
// false when this workgroup has no tile (uniform over the workgroup).
template <int GRP>
__device__ bool decode_tile(const GemmArgs& g, int ntn, int mtm, int t, int* sched, Tile& tl) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int n = lane < g.E ? g.split[lane] : 0;
        int tiles = GRP == G_M ? ((n + kGemmBM - 1) / kGemmBM) * ntn : 0;
        sched[lane] = wave_incl_scan(tiles);
        sched[64 + lane] = wave_incl_scan(n);
        sched[128 + lane] = n;
        sched[192 + lane] = wave_incl_scan((n + 31) / 32);
    }
    __syncthreads();
    int e;
    int tloc;
    if (GRP == G_M) {
        e = 0;
        while (e < g.E && sched[e] <= t) ++e;
        if (e >= g.E) return false;
        tloc = t - (e ? sched[e - 1] : 0);
        int mt = (sched[128 + e] + kGemmBM - 1) / kGemmBM;
        tl.n_tile = tloc / mt;
        tl.m0 = (tloc - tl.n_tile * mt) * kGemmBM;
    } else {
        int per = mtm * ntn;
        e = t / per;
        if (e >= g.E) return false;
        tloc = t - e * per;
        tl.n_tile = tloc / mtm;
        tl.m0 = (tloc - tl.n_tile * mtm) * kGemmBM;
    }
    tl.e = e;
    tl.n0 = tl.n_tile * (kGemmBN);
    tl.row0 = e ? sched[64 + e - 1] : 0;
    tl.rows_e = sched[128 + e];
    tl.pbase = (int64_t)(e ? sched[192 + e - 1] : 0) * 32;
    tl.pad_e = ((tl.rows_e + 31) / 32) * 32;
    return true;
}

// ---------------------------------------------------------------- operand loads
// K-contiguous operand: rows of `stride` bytes; the tile row r maps to global
// row grow(r) (clamped into [0, rows_valid)); K bytes beyond kbytes read zero.
struct KOp {
    const uint8_t* base;
    int64_t stride;
    int64_t row_first;  // global row of tile row 0 (linear map)
    int rows_valid;     // global rows that exist (for clamping)
    int64_t kbytes;
    int pair_I;         // >0: SwiGLU pairing of gate/up rows (tile covers 128 j)
    int j0;
};

__device__ __forceinline__ int64_t kop_row(const KOp& op, int r) {
    int64_t gr;
    if (op.pair_I > 0)
        gr = (int64_t)((r >> 5) & 1) * op.pair_I + op.j0 + (r >> 6) * 32 + (r & 31);
    else
        gr = op.row_first + r;
    return gr < op.rows_valid ? gr : (int64_t)op.rows_valid - 1;
}

__device__ __forceinline__ void load_kop(const KOp& op, int64_t k0b, u32x4 (&r)[4]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int id = tid + i * kGemmThreads;
        int row = id >> 3, kc = id & 7;
        int64_t kb = k0b + kc * 16;
        r[i] = (u32x4){0u, 0u, 0u, 0u};
        if (kb < op.kbytes) r[i] = *(const u32x4*)(op.base + kop_row(op, row) * op.stride + kb);
    }
}

__device__ __forceinline__ void store_kop(uint8_t* lds, const u32x4 (&r)[4]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int id = tid + i * kGemmThreads;
        *(u32x4*)(lds + lds_off(id >> 3, id & 7)) = r[i];
    }
}

// M/N-contiguous bf16 operand: element (k, mn) at base + k*stride + mn*2.
struct MNOp {
    const uint8_t* base;
    int64_t stride;
    int k_valid;
    int mn_valid;
};

__device__ __forceinline__ void load_mnop(const MNOp& op, int k0, u32x4 (&r)[4]) {
    const int tid = threadIdx.x;
    const int mc = tid & 31, kg = tid >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int k = k0 + kg * 4 + i;
        r[i] = (u32x4){0u, 0u, 0u, 0u};
        if (k < op.k_valid && mc * 8 < op.mn_valid)
            r[i] = *(const u32x4*)(op.base + (int64_t)k * op.stride + mc * 16);
    }
}

// 4 K-rows x 8 elements -> 8 LDS rows (one per element) of 4 K-values.
__device__ __forceinline__ void store_mnop(uint8_t* lds, const u32x4 (&r)[4]) {
    const int tid = threadIdx.x;
    const int mc = tid & 31, kg = tid >> 5;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
        const int w = n >> 1, sh = (n & 1) * 16;
        uint32_t e0 = (r[0][w] >> sh) & 0xffffu, e1 = (r[1][w] >> sh) & 0xffffu;
        uint32_t e2 = (r[2][w] >> sh) & 0xffffu, e3 = (r[3][w] >> sh) & 0xffffu;
        int row = mc * 8 + n;
        *(u32x2*)(lds + lds_off(row, kg >> 1) + ((kg & 1) << 3)) =
            (u32x2){e0 | (e1 << 16), e2 | (e3 << 16)};
    }
}

// MXFP8 scales of one K step (4 blocks of 32) for one tile row, as a dword
// (byte b = block 4*kt + b).  Blocks past nblk read 127 (2^0; their codes
// are zero anyway).
__device__ __forceinline__ uint32_t load_scales(const uint8_t* srow, int kt, int nblk,
                                                bool dword_ok) {
    int b0 = kt * 4;
    if (dword_ok && b0 + 4 <= nblk) return *(const uint32_t*)(srow + b0);
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        uint32_t s = b0 + b < nblk ? srow[b0 + b] : 127u;
        v |= s << (8 * b);
    }
    return v;
}

__device__ __forceinline__ float silu_f(float x) { return x / (1.f + __expf(-x)); }
__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + __expf(-x)); }

__device__ __forceinline__ float half_max32(float v) {
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float half_sum32(float v) {
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Row (along the 32 columns of a fragment) + column (along its 32 rows)
// MXFP8 quantization of one 32x32 fragment value set held in MFMA C layout.
// vals[v] is the value at row (4*(lane>>5) + 8*(v>>2) + (v&3)), column lane&31.
struct QOut {
    uint8_t* row_codes;   // + grouped row * row_ld + column
    int64_t row_ld;
    uint8_t* row_scales;  // + grouped row * (row_ld/32) + column/32
    uint8_t* col_codes;   // grouped columnwise layout base of this expert (+ pbase*C)
    uint8_t* col_scales;
    int64_t C;            // columns of the columnwise layout
};

__device__ __forceinline__ void quant_fragment(const float (&vals)[16], int64_t grow0,
                                               int frow0, int rows_e, int pad_e, int col,
                                               int64_t pbase, const QOut& q) {
    const int lane = threadIdx.x & 63;
    const int hi = lane >> 5;
    // rowwise: each row's 32 values sit in the 32 lanes of one half-wave
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        int lr = 4 * hi + 8 * (v >> 2) + (v & 3);
        float m = half_max32(__builtin_fabsf(vals[v]));
        uint32_t S = mx_scale_byte(m);
        if (frow0 + lr < rows_e) {
            int64_t gr = grow0 + lr;
            q.row_codes[gr * q.row_ld + col] = (uint8_t)mx_encode(vals[v], S);
            if ((lane & 31) == 0) q.row_scales[gr * (q.row_ld / 32) + col / 32] = (uint8_t)S;
        }
    }
    // columnwise: the fragment's 32 rows are one block (rows past the expert
    // count as zero); lane and lane^32 hold the two halves
    if (frow0 < rows_e) {
        float m = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            int lr = 4 * hi + 8 * (v >> 2) + (v & 3);
            if (frow0 + lr < rows_e) m = fmaxf(m, __builtin_fabsf(vals[v]));
        }
        m = fmaxf(m, __shfl_xor(m, 32));
        uint32_t S = mx_scale_byte(m);
        uint8_t* dst = q.col_codes + pbase * q.C + (int64_t)col * pad_e + frow0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t w = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int v = 4 * j + i;
                int lr = 4 * hi + 8 * j + i;
                float x = frow0 + lr < rows_e ? vals[v] : 0.f;
                w |= mx_encode(x, S) << (8 * i);
            }
            *(uint32_t*)(dst + 4 * hi + 8 * j) = w;
        }
        if (hi == 0)
            q.col_scales[pbase / 32 * q.C + (int64_t)col * (pad_e / 32) + frow0 / 32] = (uint8_t)S;
    } else {
        // keep the shuffle pattern uniform across the wave
        (void)__shfl_xor(0.f, 32);
    }
}

// ---------------------------------------------------------------- the kernel
template <int DT, int LA, int LB, int GRP, int EPI>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(GemmArgs g, int ntn, int mtm) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kLdsB];
    __shared__ uint32_t ssc[2][2][kGemmBM];    // MXFP8 scales [stage][A/B][row]
    __shared__ int sched[256];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;

    // XCD-aware remap: dispatch is round-robin over 8 XCDs; hand XCD x the
    // contiguous logical range [x*G/8, (x+1)*G/8).
    const int G8 = gridDim.x >> 3;
    const int t = (blockIdx.x & 7) * G8 + (blockIdx.x >> 3);

    Tile tl;
    if (!decode_tile<GRP>(g, ntn, mtm, t, sched, tl)) return;

    // ---- operand descriptors
    constexpr int kElemB = DT == DT_BF16 ? 2 : 1;
    KOp ka{}, kb{};
    MNOp ma{}, mb{};
    int64_t kext;       // K extent in elements
    const uint8_t* sa_row = nullptr;   // scale row of this thread's A/B row (MX)
    int nblk = 0;
    bool sdw = false;
    if (GRP == G_M) {
        kext = g.K;
        ka.base = (const uint8_t*)g.a;
        ka.stride = g.lda * kElemB;
        ka.row_first = tl.row0 + tl.m0;
        ka.rows_valid = (int)g.rows;
        ka.kbytes = (int64_t)g.K * kElemB;
        ka.pair_I = 0;
        if (LB == L_KMAJ) {
            kb.base = (const uint8_t*)g.b.p[tl.e];
            kb.stride = g.ldb * kElemB;
            kb.row_first = tl.n0;
            kb.rows_valid = EPI == EPI_SWIGLU_FWD ? 2 * g.I : g.N;
            kb.kbytes = (int64_t)g.K * kElemB;
            kb.pair_I = EPI == EPI_SWIGLU_FWD ? g.I : 0;
            kb.j0 = tl.n_tile * (kGemmBN / 2);
        } else {
            mb.base = (const uint8_t*)g.b.p[tl.e] + (int64_t)tl.n0 * 2;
            mb.stride = g.ldb * 2;
            mb.k_valid = g.K;
            mb.mn_valid = g.N - tl.n0;
        }
        if (DT == DT_MX) {
            nblk = g.K / 32;
            sdw = true;
            if (tid < kGemmBM) {
                int64_t r = kop_row(ka, tid);
                sa_row = g.a_scale + r * g.lda_s;
            } else {
                int64_t r = kop_row(kb, tid - kGemmBM);
                sa_row = (const uint8_t*)g.b_scale.p[tl.e] + r * g.ldb_s;
            }
        }
    } else {
        kext = DT == DT_MX ? tl.pad_e : tl.rows_e;
        if (DT == DT_BF16) {
            ma.base = (const uint8_t*)g.a + (tl.row0 * g.lda + tl.m0) * 2;
            ma.stride = g.lda * 2;
            ma.k_valid = tl.rows_e;
            ma.mn_valid = g.M - tl.m0;
            mb.base = (const uint8_t*)g.b.p[0] + (tl.row0 * g.ldb + tl.n0) * 2;
            mb.stride = g.ldb * 2;
            mb.k_valid = tl.rows_e;
            mb.mn_valid = g.N - tl.n0;
        } else {
            ka.base = (const uint8_t*)g.a + tl.pbase * g.M;
            ka.stride = tl.pad_e;
            ka.row_first = tl.m0;
            ka.rows_valid = g.M;
            ka.kbytes = tl.pad_e;
            ka.pair_I = 0;
            kb.base = (const uint8_t*)g.b.p[0] + tl.pbase * g.N;
            kb.stride = tl.pad_e;
            kb.row_first = tl.n0;
            kb.rows_valid = g.N;
            kb.kbytes = tl.pad_e;
            kb.pair_I = 0;
            nblk = tl.pad_e / 32;
            sdw = (tl.pad_e % 128) == 0;
            if (tid < kGemmBM)
                sa_row = g.a_scale + tl.pbase / 32 * g.M + kop_row(ka, tid) * (tl.pad_e / 32);
            else
                sa_row = (const uint8_t*)g.b_scale.p[0] + tl.pbase / 32 * g.N +
                         kop_row(kb, tid - kGemmBM) * (tl.pad_e / 32);
        }
    }
    constexpr int kStepElems = DT == DT_BF16 ? 64 : 128;
    const int nk = (int)((kext + kStepElems - 1) / kStepElems);

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    u32x4 ra[4], rb[4];
    uint32_t rs = 0;
    auto gload = [&](int kt) {
        if (LA == L_KMAJ) load_kop(ka, (int64_t)kt * kRowB, ra);
        else load_mnop(ma, kt * 64, ra);
        if (LB == L_KMAJ) load_kop(kb, (int64_t)kt * kRowB, rb);
        else load_mnop(mb, kt * 64, rb);
        if (DT == DT_MX) rs = load_scales(sa_row, kt, nblk, sdw);
    };
    auto sstore = [&](int st) {
        uint8_t* base = smem + st * kStageB;
        if (LA == L_KMAJ) store_kop(base, ra);
        else store_mnop(base, ra);
        if (LB == L_KMAJ) store_kop(base + kTileB, rb);
        else store_mnop(base + kTileB, rb);
        if (DT == DT_MX) ssc[st][tid >> 8][tid & 255] = rs;
    };

    if (nk > 0) {
        gload(0);
        sstore(0);
    }
    __syncthreads();

    const int fr = lane & 31, hi = lane >> 5;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        const uint8_t* A = smem + cur * kStageB;
        const uint8_t* B = A + kTileB;
        if (DT == DT_BF16) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bf16x8_t af[4], bfr[2];
#pragma unroll
                for (int fi = 0; fi < 4; ++fi)
                    af[fi] = *(const bf16x8_t*)(A + lds_off(wm * 128 + fi * 32 + fr, s * 2 + hi));
#pragma unroll
                for (int fj = 0; fj < 2; ++fj)
                    bfr[fj] = *(const bf16x8_t*)(B + lds_off(wn * 64 + fj * 32 + fr, s * 2 + hi));
#pragma unroll
                for (int fi = 0; fi < 4; ++fi)
#pragma unroll
                    for (int fj = 0; fj < 2; ++fj)
                        acc[fi][fj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fi], bfr[fj],
                                                                              acc[fi][fj], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                // Operand layout of the scaled 32x32x64 MFMA: lane (row r, half h)
                // holds K [16h, 16h+16) and [32+16h, 32+16h+16) of the 64-K step;
                // the E8M0 scale of K-block 0 of row r is taken from lane r, that
                // of block 1 from lane r+32; opsel picks the byte of the register.
                i32x8 af[4], bfr[2];
                uint32_t sa[4], sb[2];
#pragma unroll
                for (int fi = 0; fi < 4; ++fi) {
                    int row = wm * 128 + fi * 32 + fr;
                    u32x4 lo = *(const u32x4*)(A + lds_off(row, s * 4 + hi));
                    u32x4 up = *(const u32x4*)(A + lds_off(row, s * 4 + 2 + hi));
                    af[fi] = (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                     (int)up[0], (int)up[1], (int)up[2], (int)up[3]};
                    sa[fi] = ssc[cur][0][row] >> (8 * hi);
                }
#pragma unroll
                for (int fj = 0; fj < 2; ++fj) {
                    int row = wn * 64 + fj * 32 + fr;
                    u32x4 lo = *(const u32x4*)(B + lds_off(row, s * 4 + hi));
                    u32x4 up = *(const u32x4*)(B + lds_off(row, s * 4 + 2 + hi));
                    bfr[fj] = (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                      (int)up[0], (int)up[1], (int)up[2], (int)up[3]};
                    sb[fj] = ssc[cur][1][row] >> (8 * hi);
                }
#pragma unroll
                for (int fi = 0; fi < 4; ++fi)
#pragma unroll
                    for (int fj = 0; fj < 2; ++fj)
                        acc[fi][fj] = s == 0
                            ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                  af[fi], bfr[fj], acc[fi][fj], 0, 0, 0, (int)sa[fi], 0, (int)sb[fj])
                            : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                  af[fi], bfr[fj], acc[fi][fj], 0, 0, 2, (int)sa[fi], 2, (int)sb[fj]);
            }
        }
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }

    // ---------------------------------------------------------------- epilogues
    if (EPI == EPI_STORE) {
        bf16_t* C;
        int64_t ldc = g.ldc;
        int row_lim, col_lim = g.N - tl.n0;
        if (GRP == G_M) {
            C = (bf16_t*)g.c + (tl.row0 + tl.m0) * ldc + tl.n0;
            row_lim = tl.rows_e - tl.m0;
        } else {
            C = (bf16_t*)g.c_tab.p[tl.e] + (int64_t)tl.m0 * ldc + tl.n0;
            row_lim = g.M - tl.m0;
        }
#pragma unroll
        for (int fi = 0; fi < 4; ++fi)
#pragma unroll
            for (int fj = 0; fj < 2; ++fj) {
                int col = wn * 64 + fj * 32 + fr;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    int row = wm * 128 + fi * 32 + 4 * hi + 8 * (v >> 2) + (v & 3);
                    if (row < row_lim && col < col_lim)
                        C[(int64_t)row * ldc + col] = (bf16_t)f32_to_bf16(acc[fi][fj][v]);
                }
            }
        return;
    }

    if (EPI == EPI_SWIGLU_FWD) {
        // fragment fj = 0 holds gate columns, fj = 1 the up columns of the same j
        const int I = g.I;
        const int j = tl.n_tile * (kGemmBN / 2) + wn * 32 + fr;
        QOut q{g.q_row, I, g.q_row_s, g.q_col, g.q_col_s, I};
#pragma unroll
        for (int fi = 0; fi < 4; ++fi) {
            const int frow0 = tl.m0 + wm * 128 + fi * 32;   // row inside the expert
            const int64_t grow0 = tl.row0 + frow0;
            float a2v[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                int lr = 4 * hi + 8 * (v >> 2) + (v & 3);
                float gt = acc[fi][0][v], up = acc[fi][1][v];
                bool ok = frow0 + lr < tl.rows_e;
                float p = ok ? g.prob[grow0 + lr] : 0.f;
                a2v[v] = p * silu_f(gt) * up;
                if (ok) {
                    bf16_t* a1r = g.a1 + (grow0 + lr) * (2 * (int64_t)I);
                    a1r[j] = (bf16_t)f32_to_bf16(gt);
                    a1r[I + j] = (bf16_t)f32_to_bf16(up);
                    if (DT == DT_BF16) g.act[(grow0 + lr) * (int64_t)I + j] = (bf16_t)f32_to_bf16(a2v[v]);
                }
            }
            if (DT == DT_MX) quant_fragment(a2v, grow0, frow0, tl.rows_e, tl.pad_e, j, tl.pbase, q);
        }
        return;
    }

    if (EPI == EPI_SWIGLU_BWD) {
        const int I = g.I;
        float* red = (float*)smem;                     // [4 waves along N][256 rows]
        float rowpart[4][16];
        QOut q{g.q_row, 2 * (int64_t)I, g.q_row_s, g.q_col, g.q_col_s, 2 * (int64_t)I};
#pragma unroll
        for (int fi = 0; fi < 4; ++fi)
#pragma unroll
            for (int v = 0; v < 16; ++v) rowpart[fi][v] = 0.f;
#pragma unroll
        for (int fj = 0; fj < 2; ++fj) {
            const int j = tl.n0 + wn * 64 + fj * 32 + fr;
            const bool jok = j < I;
#pragma unroll
            for (int fi = 0; fi < 4; ++fi) {
                const int frow0 = tl.m0 + wm * 128 + fi * 32;
                const int64_t grow0 = tl.row0 + frow0;
                float dgv[16], duv[16];
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    int lr = 4 * hi + 8 * (v >> 2) + (v & 3);
                    bool ok = jok && (frow0 + lr < tl.rows_e);
                    float d = acc[fi][fj][v];
                    float gt = 0.f, up = 0.f, p = 0.f;
                    if (ok) {
                        const bf16_t* a1r = g.a1 + (grow0 + lr) * (2 * (int64_t)I);
                        gt = bf16_to_f32(a1r[j]);
                        up = bf16_to_f32(a1r[I + j]);
                        p = g.prob[grow0 + lr];
                    }
                    float sg = sigmoid_f(gt);
                    float sl = gt * sg;
                    float dp = d * p;
                    dgv[v] = dp * up * sg * (1.f + gt * (1.f - sg));
                    duv[v] = dp * sl;
                    rowpart[fi][v] += ok ? d * sl * up : 0.f;
                    if (DT == DT_BF16 && ok) {
                        bf16_t* o = g.act + (grow0 + lr) * (2 * (int64_t)I);
                        o[j] = (bf16_t)f32_to_bf16(dgv[v]);
                        o[I + j] = (bf16_t)f32_to_bf16(duv[v]);
                    }
                }
                if (DT == DT_MX && tl.n0 + wn * 64 + fj * 32 < I) {
                    quant_fragment(dgv, grow0, frow0, tl.rows_e, tl.pad_e, j, tl.pbase, q);
                    quant_fragment(duv, grow0, frow0, tl.rows_e, tl.pad_e, I + j, tl.pbase, q);
                }
            }
        }
        // probability gradient: sum over this tile's columns, per row
#pragma unroll
        for (int fi = 0; fi < 4; ++fi)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                float sm = half_sum32(rowpart[fi][v]);
                int row = wm * 128 + fi * 32 + 4 * hi + 8 * (v >> 2) + (v & 3);
                if (fr == 0) red[wn * kGemmBM + row] = sm;
            }
        __syncthreads();
        if (tid < kGemmBM) {
            int row = tid;
            if (tl.m0 + row < tl.rows_e) {
                float sm = red[row] + red[kGemmBM + row] + red[2 * kGemmBM + row] +
                           red[3 * kGemmBM + row];
                g.dprob_part[(tl.row0 + tl.m0 + row) * (int64_t)ntn + tl.n_tile] = sm;
            }
        }
        return;
    }
}

__global__ void dprob_reduce_kernel(const float* __restrict__ part, int64_t rows, int ntiles,
                                    float* __restrict__ dprob) {
    int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= rows) return;
    float s = 0.f;
    for (int n = 0; n < ntiles; ++n) s += part[r * ntiles + n];
    dprob[r] = s;
}

// ---------------------------------------------------------------- launcher
int gemm_n_tiles(int epi, int N, int I) {
    if (epi == EPI_SWIGLU_FWD) return I / (kGemmBN / 2);
    if (epi == EPI_SWIGLU_BWD) return (I + kGemmBN - 1) / kGemmBN;
    return (N + kGemmBN - 1) / kGemmBN;
}

template <int DT, int LA, int LB, int GRP, int EPI>
static hipError_t run(const GemmArgs& g, hipStream_t s) {
    const int ntn = gemm_n_tiles(EPI, g.N, g.I);
    int mtm = 0;
    int64_t tiles;
    if (GRP == G_M) {
        // upper bound of sum_e ceil(M_e / BM)
        int64_t mt = (g.rows + (int64_t)g.E * (kGemmBM - 1)) / kGemmBM;
        tiles = mt * ntn;
    } else {
        mtm = (g.M + kGemmBM - 1) / kGemmBM;
        tiles = (int64_t)g.E * mtm * ntn;
    }
    if (tiles == 0) return hipSuccess;
    int64_t grid = (tiles + 7) / 8 * 8;
    TraceScope ts(g.name ? g.name : "gemm", s);
    gemm_kernel<DT, LA, LB, GRP, EPI><<<(unsigned)grid, kGemmThreads, 0, s>>>(g, ntn, mtm);
    return hipGetLastError();
}

hipError_t launch_gemm(int dtype, int la, int lb, int grp, int epi, const GemmArgs& g,
                       hipStream_t s) {
#define MOE_GEMM_CASE(DT, LA, LB, GRP, EPI)                                        \
    if (dtype == DT && la == LA && lb == LB && grp == GRP && epi == EPI)           \
        return run<DT, LA, LB, GRP, EPI>(g, s);
    // bf16
    MOE_GEMM_CASE(DT_BF16, L_KMAJ, L_KMAJ, G_M, EPI_SWIGLU_FWD)
    MOE_GEMM_CASE(DT_BF16, L_KMAJ, L_KMAJ, G_M, EPI_STORE)
    MOE_GEMM_CASE(DT_BF16, L_KMAJ, L_MNMAJ, G_M, EPI_SWIGLU_BWD)
    MOE_GEMM_CASE(DT_BF16, L_KMAJ, L_MNMAJ, G_M, EPI_STORE)
    MOE_GEMM_CASE(DT_BF16, L_MNMAJ, L_MNMAJ, G_K, EPI_STORE)
    // mxfp8
    MOE_GEMM_CASE(DT_MX, L_KMAJ, L_KMAJ, G_M, EPI_SWIGLU_FWD)
    MOE_GEMM_CASE(DT_MX, L_KMAJ, L_KMAJ, G_M, EPI_STORE)
    MOE_GEMM_CASE(DT_MX, L_KMAJ, L_KMAJ, G_M, EPI_SWIGLU_BWD)
    MOE_GEMM_CASE(DT_MX, L_KMAJ, L_KMAJ, G_K, EPI_STORE)
#undef MOE_GEMM_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_dprob_reduce(const float* part, int64_t rows, int ntiles, float* dprob,
                               hipStream_t s) {
    if (rows == 0) return hipSuccess;
    TraceScope ts("dprob_reduce", s);
    dprob_reduce_kernel<<<(unsigned)((rows + 255) / 256), 256, 0, s>>>(part, rows, ntiles, dprob);
    return hipGetLastError();
}

}  // namespace moe
