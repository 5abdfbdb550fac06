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
//   * 256 x 256 output tile per workgroup of 256 threads (4 waves, 2 x 2);
//     every wave owns a 128 x 128 sub-tile = 4 x 4 MFMA 32x32 fragments whose
//     256 fp32 accumulators live in the accumulation registers (one wave per
//     SIMD, 512 registers per lane).
//   * K steps of 64 bytes per operand row: 32 bf16 (2 x
//     v_mfma_f32_32x32x16_bf16) or 64 E4M3 (one
//     v_mfma_scale_f32_32x32x64_f8f6f4, the E8M0 scale of every 32 K-values
//     and row fed straight to the instruction, so nothing is dequantized).
//   * LDS holds four stages of both operand tiles (4 x 32 KiB); the loads of
//     steps k+1..k+3 are in flight while step k feeds the MFMAs, one barrier
//     per step.  Operands go from memory to LDS without passing through
//     registers (buffer_load_dwordx4 ... lds: lane l's 16 bytes land at the
//     wave's LDS base + 16 l, so the lane picks the global chunk that fills
//     its slot); 16-byte chunks of a 64-byte tile row are XOR-swizzled by
//     (row >> 2) & 3 so fragment reads of 16 consecutive rows hit distinct
//     banks.  Offsets past a row's valid K read zeros.  The fragments of
//     step k+1 are read from LDS into a second register set right after the
//     barrier that publishes them, under the last MFMAs of step k.
//   * Epilogues: each wave stages its 128 x 128 result through its own LDS
//     region, 32 rows at a time (last slice first), and syncs only on its
//     own LDS accesses.  Outputs that a wave owns whole lines of (the plain
//     stores, the saved A1, bf16 dA1) leave in whole 128-byte lines with
//     streaming stores.
//   * M/N-contiguous bf16 operands (the dgrad weights and both weight-gradient
//     operands) are staged in LDS in their natural [k][m] order (16-byte
//     chunks of a 512-byte row XOR-ed with 4*(k&3)) and turned into K-packed
//     MFMA fragments by ds_read_b64_tr_b16, which transposes 4 K-rows x 16
//     columns across each 16-lane group, so no transposed copy is written.
//   * MXFP8 operands carry block-major scales ([K/32][rows]); one dword per
//     lane of one wave moves the 256 scale bytes of a block.
//   * Grouping: the tile list is the concatenation over experts of their
//     tiles (ragged M: ceil(M_e / 256) x N-tiles each; ragged K: a fixed
//     M x N grid each, looping over the expert's rows).  The per-expert prefix
//     sums are rebuilt on the device from split_sizes by the first wave of
//     every workgroup.  Tiles are spread over the 8 XCDs (round-robin
//     dispatch) so that all XCDs work on the same expert at the same time,
//     each on its own N-tiles, in bands of row-tiles that share an L2.
//   * No float atomics: the probability gradient is written as per-(row,
//     N-tile) partial sums and reduced in a fixed order by a second kernel.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "mlp.hpp"
#include "trace.hpp"

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

constexpr int kStages = 4;                    // LDS pipeline depth (loads run 3 steps ahead)
constexpr int kRowB = 64;                     // K-contiguous LDS tile row (bytes per K step)
constexpr int kTileB = kGemmBM * kRowB;       // 16 KiB per operand per stage
constexpr int kStageB = 2 * kTileB;           // A + B
constexpr int kLdsB = kStages * kStageB;      // 128 KiB
constexpr int kMNRowB = kGemmBM * 2;          // M/N-contiguous LDS row: 256 bf16 = 512 B
constexpr uint32_t kOob = 0x80000000u;        // buffer offset that reads zeros

// K-contiguous tile: row r, 16-byte chunk c (4 per row); XOR with (r>>2)&3
// makes the 16-byte reads of 16 consecutive rows hit 16 distinct bank groups.
__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * kRowB + ((chunk ^ ((row >> 2) & 3)) << 4);
}
// M/N-contiguous tile: K row k (32 per stage), 16-byte chunk c (32 per row)
__device__ __forceinline__ int mn_off(int k, int c) {
    return k * kMNRowB + ((c ^ ((k & 3) << 2)) << 4);
}

// Per-workgroup tile descriptor.
struct Tile {
    int e;           // expert
    int m0, n0;      // first row (inside the expert for G_M) / column of the tile
    int64_t row0;    // first grouped row of the expert
    int rows_e;      // M_e (= K extent for G_K)
    int64_t pbase;   // sum of the padded (32) sizes of earlier experts
    int pad_e;       // padded size of this expert
    int64_t pbase64; // the same sums with sizes padded to 64 (row-pair grouped layouts)
    int pad64_e;
    int n_tile;
};

// Order of the mt x nt tiles of one expert: bands of kGroupM row-tiles, and
// inside a band the row-tiles vary fastest.  Consecutive workgroups (which
// run together on one XCD) then share both operands: each weight tile is read
// by up to kGroupM concurrent tiles and each activation tile by the band's
// column-tiles in flight.
constexpr int kGroupM = 8;
__device__ __forceinline__ void grouped_order(int t, int mt, int nt, int& m, int& n) {
    int band = t / (kGroupM * nt);
    int m0 = band * kGroupM;
    int gm = min(mt - m0, kGroupM);
    int r = t - band * kGroupM * nt;
    m = m0 + r % gm;
    n = r / gm;
}

// Builds the per-expert prefix tables in LDS and decodes the tile.  Returns
// false when this workgroup has no tile (uniform over the workgroup).
// sched: [0, 64) tile prefix, [64, 128) row prefix, [128, 192) rows,
// [192, 256) and [256, 320) prefixes of the 32- and 64-padded sizes,
// [320, 384) the weight gradients' expert order.
template <int GRP>
__device__ bool decode_tile(const GemmArgs& g, int ntn, int mtm, int t, int* sched, Tile& tl) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const int n = clamp_group_size(lane < g.E ? g.split[lane] : 0, g.rows);
        int tiles = GRP == G_M ? ((n + kGemmBM - 1) / kGemmBM) * ntn : 0;
        sched[lane] = wave_incl_scan(tiles);
        sched[64 + lane] = wave_incl_scan(n);
        sched[128 + lane] = n;
        sched[192 + lane] = wave_incl_scan((n + 31) / 32);
        sched[256 + lane] = wave_incl_scan((n + 63) / 64);
        if (GRP == G_K) {
            // weight gradients: experts in decreasing order of rows (ties by
            // index), so the longest tiles start first and the short ones fill
            // in behind them instead of trailing at the end of the grid
            int rank = 0;
            for (int j = 0; j < g.E; ++j) {
                const int m = __shfl(n, j);
                rank += (m > n || (m == n && j < lane)) ? 1 : 0;
            }
            if (lane < g.E) sched[320 + rank] = lane;
        }
    }
    __syncthreads();
    int e;
    int tloc;
    if (GRP == G_K && (mtm & 7) == 0 && g.M > g.N) {
        // Weight gradient whose first operand is the larger one (dW1 = dA1^T
        // Xp: 2I rows against H): XCD x takes the row tiles m = 8m' + x of
        // every expert, so each XCD reads its own eighth of that operand once
        // and only the smaller one is read by all XCDs.
        const int x = blockIdx.x & 7, i = blockIdx.x >> 3, mt8 = mtm >> 3;
        const int per = mt8 * ntn;
        const int q = i / per;
        if (q >= g.E) return false;
        e = sched[320 + q];
        tloc = i - q * per;
        int m8;
        grouped_order(tloc, mt8, ntn, m8, tl.n_tile);
        tl.m0 = (m8 * 8 + x) * kGemmBM;
    } else if ((ntn & 7) == 0) {
        // Expert-synchronous split over the 8 XCDs: XCD x takes the N-tiles
        // n = 8n' + x of every expert, experts in order, so that all XCDs
        // stream the same expert at the same time: the activation rows they
        // all read are fetched from HBM once and served to the other XCDs by
        // the last-level cache, and every weight byte comes from HBM once.
        // Inside the XCD's share: bands of row-tiles (grouped_order).
        const int x = blockIdx.x & 7, i = blockIdx.x >> 3, nt8 = ntn >> 3;
        int mt;
        if (GRP == G_M) {
            e = 0;
            while (e < g.E && (sched[e] >> 3) <= i) ++e;
            if (e >= g.E) return false;
            tloc = i - (e ? (sched[e - 1] >> 3) : 0);
            mt = (sched[128 + e] + kGemmBM - 1) / kGemmBM;
        } else {
            const int per = mtm * nt8;
            const int q = i / per;
            if (q >= g.E) return false;
            e = sched[320 + q];
            tloc = i - q * per;
            mt = mtm;
        }
        int m, n8;
        grouped_order(tloc, mt, nt8, m, n8);
        tl.n_tile = n8 * 8 + x;
        tl.m0 = m * kGemmBM;
    } else if (GRP == G_M) {
        e = 0;
        while (e < g.E && sched[e] <= t) ++e;
        if (e >= g.E) return false;
        tloc = t - (e ? sched[e - 1] : 0);
        int mt = (sched[128 + e] + kGemmBM - 1) / kGemmBM;
        int m;
        grouped_order(tloc, mt, ntn, m, tl.n_tile);
        tl.m0 = m * kGemmBM;
    } else {
        int per = mtm * ntn;
        const int q = t / per;
        if (q >= g.E) return false;
        e = sched[320 + q];
        tloc = t - q * per;
        int m;
        grouped_order(tloc, mtm, ntn, m, tl.n_tile);
        tl.m0 = m * kGemmBM;
    }
    // every field is the same for the whole workgroup: say so, so that the
    // address arithmetic built on them stays in scalar registers
    tl.e = __builtin_amdgcn_readfirstlane(e);
    tl.m0 = __builtin_amdgcn_readfirstlane(tl.m0);
    tl.n_tile = __builtin_amdgcn_readfirstlane(tl.n_tile);
    tl.n0 = tl.n_tile * kGemmBN;
    tl.row0 = __builtin_amdgcn_readfirstlane(e ? sched[64 + e - 1] : 0);
    tl.rows_e = __builtin_amdgcn_readfirstlane(sched[128 + e]);
    tl.pbase = (int64_t)__builtin_amdgcn_readfirstlane(e ? sched[192 + e - 1] : 0) * 32;
    tl.pad_e = ((tl.rows_e + 31) / 32) * 32;
    tl.pbase64 = (int64_t)__builtin_amdgcn_readfirstlane(e ? sched[256 + e - 1] : 0) * 64;
    tl.pad64_e = ((tl.rows_e + 63) / 64) * 64;
    return true;
}

// ---------------------------------------------------------------- operand loads
// K-contiguous operand from `base`: tile row r maps to operand row kop_row(r)
// (clamped into [0, rows_valid)); K bytes at or past kbytes read zero.  bf16
// operands are row-major with rows of `stride` bytes; 8-bit operands are in
// the row-pair layout (common.hpp) with `stride` bytes per row pair, so the
// 16 lanes that fill two neighbouring tile rows fetch one whole 128-byte line.
// The bases are taken per tile (and per expert), so offsets from them stay
// below 2^31.
struct KOp {
    const uint8_t* base;
    int64_t stride;
    int row_first;      // operand row of tile row 0 (linear map)
    int rows_valid;     // operand rows that exist (for clamping)
    int kbytes;
    int pair_I;         // >0: SwiGLU pairing of gate/up rows (tile covers 128 j)
    int j0;
};

__device__ __forceinline__ int kop_row(const KOp& op, int r) {
    int gr;
    if (op.pair_I > 0)
        gr = ((r >> 5) & 1) * op.pair_I + op.j0 + (r >> 6) * 32 + (r & 31);
    else
        gr = op.row_first + r;
    return gr < op.rows_valid ? gr : op.rows_valid - 1;
}

// LDS-DMA issued through inline assembly.  The compiler does not see these
// loads, so it inserts no waits for them (it cannot track many in-flight
// LDS-DMA stores and would otherwise wait for all of them before every LDS
// read); the pipeline waits for them explicitly with pipe_barrier.  The
// buffer resource (base, stride 0, 2^31-1 records) makes offsets >= 2^31 read
// zeros.  buffer_load_dwordx4 ... lds writes lane l's 16 bytes at M0 + 16 l;
// buffer_load_dword ... lds writes lane l's 4 bytes at M0 + 4 l.
typedef __attribute__((ext_vector_type(4))) int i32x4;

__device__ __forceinline__ i32x4 make_rsrc(const void* p) {
    uint64_t a = (uint64_t)p;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    r[2] = 0x7fffffff;
    r[3] = 0x00020000;
    return r;
}

// LDS byte address of a shared-memory pointer (the low 32 bits of the
// generic address; the LDS aperture is 4 GiB aligned), as a uniform value.
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

__device__ __forceinline__ void dma16(const i32x4& rs, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 ::"s"(lds), "v"(voff), "s"(rs) : "memory");
}

__device__ __forceinline__ void dma4(const i32x4& rs, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 ::"s"(lds), "v"(voff), "s"(rs) : "memory");
}

// Pipeline barrier: wait until at most N vector-memory loads (LDS-DMA batches
// of later K steps) are outstanding and all LDS accesses are done, then
// synchronize the workgroup.  __syncthreads() would also fence global memory,
// which waits for every outstanding load and so drains the look-ahead.
// The compiler does not see the waits inside the asm: the trailing
// s_waitcnt lgkmcnt(0) (free, the counter is already zero) tells it that
// every earlier LDS read has completed, so it does not hold back the MFMAs
// after the barrier for reads that landed long ago.
template <int N>
__device__ __forceinline__ void pipe_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt(63) expcnt(7) lgkmcnt(0)
}

// LDS-DMA of one K step of a K-contiguous tile: the wave's 4 instructions
// cover tile rows (wave*4 + j)*16 .. +15; slot i of instruction j is tile row
// (wave*4 + j)*16 + i/4 and physical chunk i%4, whose logical chunk is
// (i%4) ^ ((row>>2)&3) = (i%4) ^ ((i>>4)&3).
template <bool P2>
__device__ __forceinline__ void dma_kop(const KOp& op, const i32x4& rs, int k0b, uint8_t* lds) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lc16 = ((lane & 3) ^ ((lane >> 4) & 3)) << 4;    // logical 16-byte chunk
    const int kc16 = lc16 + k0b;
    const uint32_t l0 = lds_u32(lds + wave * 4 * 1024);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        int r = (wave * 4 + j) * 16 + (lane >> 2);
        const int gr = kop_row(op, r);
        uint32_t o = kOob;
        if (kc16 < op.kbytes) {
            if (P2)   // K step k0b / 64 of row pair gr / 2: line k0b / 64, half gr & 1
                o = (uint32_t)(gr >> 1) * (uint32_t)op.stride + (uint32_t)(2 * k0b) +
                    (uint32_t)((gr & 1) * 64 + lc16);
            else
                o = (uint32_t)((int64_t)gr * op.stride) + (uint32_t)kc16;
        }
        dma16(rs, o, l0 + j * 1024);
    }
}

// M/N-contiguous bf16 operand: element (k, mn) at base + k*stride + mn*2.
struct MNOp {
    const uint8_t* base;
    int64_t stride;
    int k_valid;
    int mn_valid;
};

// LDS-DMA of one K step (32 K rows x 256 columns) of an M/N-contiguous tile
// into its natural order: instruction j of the wave covers K rows
// (wave*4 + j)*2 .. +1; slot i is K row (wave*4+j)*2 + i/32, physical chunk
// i%32, logical chunk (i%32) ^ ((k&3)<<2).  Rows past k_valid and columns
// past mn_valid read zeros.  The buffer resource is rebuilt at the step's
// first K row, so offsets stay below 32 rows whatever the K extent.
__device__ __forceinline__ void dma_mnop(const MNOp& op, int k0, uint8_t* lds) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const i32x4 rs = make_rsrc(op.base + (int64_t)k0 * op.stride);
    const uint32_t l0 = lds_u32(lds + wave * 4 * 1024);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        int k = (wave * 4 + j) * 2 + (lane >> 5);
        int c = (lane & 31) ^ ((k & 3) << 2);
        bool ok = k0 + k < op.k_valid && c * 8 < op.mn_valid;
        uint32_t o = ok ? (uint32_t)(k * op.stride) + (uint32_t)(c * 16) : kOob;
        dma16(rs, o, l0 + j * 1024);
    }
}

// K-packed bf16 fragment (8 K-values, K sub-step s, columns colbase..+31) of
// an M/N-contiguous LDS tile, via two transposing reads: in each 16-lane
// group g, lane q supplies (K row kb + q/4, columns n..n+3) and receives
// column n0 + q for 4 consecutive K rows.
__device__ __forceinline__ bf16x8_t mn_frag(const uint8_t* lds, int s, int colbase) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, q = lane & 15;
    const int kb = 16 * s + 8 * (g >> 1) + (q >> 2);
    const int n = colbase + 16 * (g & 1) + 4 * (q & 3);       // element column
    const int c = n >> 3, sub = (n & 7) * 2;                   // 16-byte chunk, byte in chunk
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(lds + mn_off(kb, c) + sub));
    i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4_t*)(lds + mn_off(kb + 4, c) + sub));
    i16x8 v = {lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
    return __builtin_bit_cast(bf16x8_t, v);
}

// MXFP8 scales of one K step.  GEMM operands keep their E8M0 scales
// block-major ([block][row]), so the scales of one K block for the 256 tile
// rows are 256 bytes: one dword per lane covers 4 consecutive tile rows.
// Wave w loads operand w/2, block 2kt + (w&1), into dst[w/2][w&1][256 rows].
// off_a/off_b: offset of this lane's 4-row group inside a block row, or kOob
// when the whole group lies past the operand's rows; blocks at or past nblk
// read zero (a finite scale; their codes are zero too).
__device__ __forceinline__ void dma_scales(const i32x4& rs_a, const i32x4& rs_b,
                                           uint32_t off_a, uint32_t off_b, uint32_t ld_a,
                                           uint32_t ld_b, int kt, int nblk,
                                           uint8_t (*dst)[2][kGemmBM]) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform
    const int op = wave >> 1, blk = 2 * kt + (wave & 1);
    const uint32_t off = op ? off_b : off_a, ld = op ? ld_b : ld_a;
    const uint32_t o = (blk < nblk && off != kOob) ? (uint32_t)blk * ld + off : kOob;
    dma4(op ? rs_b : rs_a, o, lds_u32(&dst[op][wave & 1][0]));
}

// The reciprocal is the hardware's (about 1 ulp), not an IEEE division: the
// results are rounded to bf16 or E4M3 right after.
__device__ __forceinline__ float sigmoid_f(float x) {
    return __builtin_amdgcn_rcpf(1.f + __expf(-x));
}
__device__ __forceinline__ float silu_f(float x) { return x * sigmoid_f(x); }

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

// ---------------------------------------------------------------- epilogue staging
// The SwiGLU epilogues stage each 32-row slice of a wave's 128x128 result
// through a private 32 x 128 fp32 LDS region (16-byte chunks XOR-swizzled by
// row & 7), so that global traffic is 16-byte row / column pieces and the
// MXFP8 block maxima are per-lane reductions:
//   phase 1  the wave writes its 4 fragments of row slice fi;
//   phase 2  lane (row = lane/2, half = lane&1) handles 32-column blocks of
//            one row: SwiGLU math, bf16 stores, rowwise MXFP8 (codes + scale);
//   phase 3  lane = column: the 32 rows of one column -> columnwise MXFP8.
// The epilogues stage through each wave's own LDS region: between their
// phases a wave only waits for its own LDS accesses (a workgroup barrier
// would make the four waves run their store bursts in lockstep).  The empty
// asm's memory clobber also keeps the compiler from moving LDS accesses
// across it.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ int st_idx(int row, int col) {
    return row * 128 + ((((col >> 2) ^ (row & 7))) << 2) + (col & 3);
}

// Value v of a lane's 32x32 fragment is row 4*hi + 8*(v>>2) + (v&3), column
// fr.  Its row & 7 is 4*hi + (v&3), so st_idx(row, 32f + fr) is one of four
// per-lane bases plus 1024*(v>>2) + 32*f: every write takes an immediate
// offset instead of its own swizzle arithmetic.
__device__ __forceinline__ void stage_fragments(float* R, const f32x16& f0, const f32x16& f1,
                                                const f32x16& f2, const f32x16& f3,
                                                int lane = threadIdx.x & 63) {
    const int fr = lane & 31, hi = lane >> 5;
    float* base[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) base[r] = R + st_idx(4 * hi + r, fr);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        float* b = base[v & 3] + 1024 * (v >> 2);
        b[0] = f0[v];
        b[32] = f1[v];
        b[64] = f2[v];
        b[96] = f3[v];
    }
}

// bf16 staging of one 32-row slice for the plain-store epilogue: dword
// (p, c) holds rows 2p and 2p+1 of column c (low and high halves), at
// p * 128 + c.  A lane's fragment values 4g+j (rows 4hi + 8g + j) pair up as
// j = 0,1 (row pair 2hi + 4g) and j = 2,3 (row pair 2hi + 4g + 1).
__device__ __forceinline__ void stage_pairs_bf16(uint32_t* P, const f32x16& f0, const f32x16& f1,
                                                 const f32x16& f2, const f32x16& f3, int lane) {
    const int fr = lane & 31, hi = lane >> 5;
    uint32_t* b = P + (2 * hi) * 128 + fr;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int v = 4 * g + 2 * h;
            uint32_t* d = b + (4 * g + h) * 128;
            d[0] = pack_bf16x2(f0[v], f0[v + 1]);
            d[32] = pack_bf16x2(f1[v], f1[v + 1]);
            d[64] = pack_bf16x2(f2[v], f2[v + 1]);
            d[96] = pack_bf16x2(f3[v], f3[v + 1]);
        }
}

__device__ __forceinline__ void load_row8(const float* R, int row, int col, float (&x)[8]) {
    float4 a = *(const float4*)(R + st_idx(row, col));
    float4 b = *(const float4*)(R + st_idx(row, col + 4));
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ void store_row8(float* R, int row, int col, const float* x) {
    *(float4*)(R + st_idx(row, col)) = make_float4(x[0], x[1], x[2], x[3]);
    *(float4*)(R + st_idx(row, col + 4)) = make_float4(x[4], x[5], x[6], x[7]);
}

__device__ __forceinline__ u32x4 pack8_bf16(const float* x) {
    return (u32x4){pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                   pack_bf16x2(x[6], x[7])};
}

__device__ __forceinline__ void unpack8_bf16(u32x4 w, float* x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = lo_bf16(w[i]);
        x[2 * i + 1] = hi_bf16(w[i]);
    }
}

// One block of 32 values -> E8M0 scale and 32 E4M3 codes as two 16-byte words.
__device__ __forceinline__ uint32_t quant32(const float* x, u32x4& c0, u32x4& c1) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) m = fmaxf(m, __builtin_fabsf(x[i]));
    uint32_t S = mx_scale_byte(m);
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        uint32_t word = mx_encode4(x[4 * w], x[4 * w + 1], x[4 * w + 2], x[4 * w + 3], S);
        if (w < 4) c0[w] = word;
        else c1[w - 4] = word;
    }
    return S;
}

// Columnwise MXFP8 of column `col` of the staged region (32 rows; the
// callers stage zeros for the rows past the expert, so all 32 are read
// unconditionally) into the grouped columnwise layout.
__device__ __forceinline__ void col_quant(const float* R, int col, uint8_t* codes,
                                          uint8_t* scale) {
    float x[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) x[r] = R[st_idx(r, col)];
    u32x4 c0, c1;
    uint32_t S = quant32(x, c0, c1);
    ((u32x4*)codes)[0] = c0;
    ((u32x4*)codes)[1] = c1;
    *scale = (uint8_t)S;
}

struct EpiCtx {
    const GemmArgs& g;
    const Tile& tl;
    int wm, wn, ntn;
    float pr[4];        // routing probability of the lane's row (lane / 2) in each slice
    int lane;           // lane index (lane_after_loop)
};

// ScaledSwiGLU forward of row slice fi of the wave's tile.  Staged columns
// [64q, 64q+32) are gate and [64q+32, 64q+64) up for j = tile j0 + (2wn+q)*32.
// Largest |bf16| bit pattern of the two values in a packed word, merged into m.
__device__ __forceinline__ uint32_t max_abs_bf16x2(uint32_t m, uint32_t w) {
    return max(m, max(w & 0x7fffu, (w >> 16) & 0x7fffu));
}

template <int DT>
__device__ __forceinline__ void swiglu_fwd_rows(const EpiCtx& c, float* R, const f32x16& f0,
                                                const f32x16& f1, const f32x16& f2,
                                                const f32x16& f3, int fi, uint32_t& amx) {
    const GemmArgs& g = c.g;
    const Tile& tl = c.tl;
    const int lane = c.lane;
    const int64_t I = g.I;
    stage_fragments(R, f0, f1, f2, f3, lane);
    wave_lds_sync();
    const int frow0 = tl.m0 + c.wm * 128 + fi * 32;      // row inside the expert
    const int valid = min(32, tl.rows_e - frow0);          // rows of this slice that exist
    {
        // A1, gate and up of the wave's 64 j: 8 lanes write one row's
        // 128-byte line, 8 rows per instruction, streamed past L2 (whole
        // lines, read again only by the backward)
        const int c8 = lane & 7;
        const int64_t jw0 = tl.n_tile * (kGemmBN / 2) + 2 * c.wn * 32 + 8 * c8;
        const int scol = 64 * (c8 >> 2) + 8 * (c8 & 3);   // staged column of the 8 gate values
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = (lane >> 3) + 8 * i;
            if (row < valid) {
                const int64_t gr = tl.row0 + frow0 + row;
                float x[8];
                load_row8(R, row, scol, x);
                __builtin_nontemporal_store(pack8_bf16(x), (u32x4*)(g.a1 + gr * 2 * I + jw0));
                load_row8(R, row, scol + 32, x);
                __builtin_nontemporal_store(pack8_bf16(x), (u32x4*)(g.a1 + gr * 2 * I + I + jw0));
            }
        }
    }
    {
        const int row = lane >> 1, q = lane & 1;
        const int j0 = tl.n_tile * (kGemmBN / 2) + (2 * c.wn + q) * 32;
        float a2[32];
        if (row < valid) {
            const int64_t gr = tl.row0 + frow0 + row;
            const float p = c.pr[fi];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                float gt[8], up[8];
                load_row8(R, row, 64 * q + 8 * b, gt);
                load_row8(R, row, 64 * q + 32 + 8 * b, up);
#pragma unroll
                for (int i = 0; i < 8; ++i) a2[8 * b + i] = p * silu_f(gt[i]) * up[i];
            }
            if (DT != DT_MX) {          // bf16 A2 (BF16, and FP8: cast later)
                u32x4* o = (u32x4*)(g.act + gr * I + j0);
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const u32x4 pk = pack8_bf16(a2 + 8 * b);
                    o[b] = pk;
                    if (DT == DT_FP8)   // the tensor maximum of the cast that follows
#pragma unroll
                        for (int q = 0; q < 4; ++q) amx = max_abs_bf16x2(amx, pk[q]);
                }
            } else {
                // rowwise codes in the row-pair layout, the row at its
                // expert-padded position
                u32x4 c0, c1;
                uint32_t S = quant32(a2, c0, c1);
                const int64_t rp = tl.pbase + frow0 + row;
                u32x4* o = (u32x4*)(g.q_row + p2_off(rp, j0, p2_stride(I)));
                o[0] = c0;
                o[1] = c1;
                g.q_row_s[(j0 / 32) * g.rows_pad + rp] = (uint8_t)S;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 32; ++i) a2[i] = 0.f;
        }
        if (DT == DT_MX)
#pragma unroll
            for (int b = 0; b < 4; ++b) store_row8(R, row, 64 * q + 8 * b, a2 + 8 * b);
    }
    wave_lds_sync();
    if (DT == DT_MX && valid > 0) {
        const int q = lane >> 5, jj = lane & 31;
        const int64_t j = tl.n_tile * (kGemmBN / 2) + (2 * c.wn + q) * 32 + jj;
        col_quant(R, 64 * q + jj, g.q_col + tl.pbase64 * I + p2_off(j, frow0, 2 * tl.pad64_e),
                  g.q_col_s + tl.pbase / 32 * I + (frow0 / 32) * I + j);
    }
    wave_lds_sync();
}

// The saved gate/up values of a backward slice (32 rows, the wave's 128 j),
// read in whole 128-byte lines (8 lanes per line of a row, streamed past L2)
// and staged as (gate, up) bf16 pairs, one pair per fp32 slot of R2, where
// the row-per-lane arithmetic reads them.  Rows past the expert stage zeros.
// load_a1 only issues the loads: the first slice's right after the K loop,
// each next slice's as soon as the current one is staged, so that they are
// in flight through a whole slice of work instead of stalling its start.
// (float4 accesses throughout, like the du stores that later reuse the
// slots, so the compiler keeps their order.)
struct A1Words { u32x4 g[4][2], u[4][2]; };

__device__ __forceinline__ void load_a1(const GemmArgs& g, const Tile& tl, int wm, int wn, int fi,
                                        int lane, A1Words& w) {
    const int64_t I = g.I;
    const int frow0 = tl.m0 + wm * 128 + fi * 32;
    const int valid = max(0, min(32, tl.rows_e - frow0));
    const int jw = tl.n0 + wn * 128;
    const bool slab = jw < I;
    // One buffer resource per slice, based at its first row: rows past the
    // expert (and every row, for a wave whose columns lie past I) are out of
    // its range and read zero, with no per-row branches or zero fills.
    // (every field is uniform: readfirstlane says so, else the compiler
    // wraps each load in a loop over the distinct descriptors of the wave)
    const int rowb = (int)(4 * I);                             // bytes per A1 row (2I bf16)
    // (readfirstlane returns int: both halves go through uint32_t, so the
    // low half is not sign-extended into the high one)
    const uint64_t base = (uint64_t)(g.a1 + (tl.row0 + frow0) * 2 * I);
    const uint32_t blo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base);
    const uint32_t bhi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32));
    const uint64_t ubase = ((uint64_t)bhi << 32) | (uint64_t)blo;
    const int nrec = __builtin_amdgcn_readfirstlane(slab ? valid * rowb : 0);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)ubase, (short)0, nrec, 0x00020000);
    const int voff = (lane >> 3) * rowb + (jw + 8 * (lane & 7)) * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int o = voff + 8 * i * rowb + 128 * s;           // row lane/8 + 8i
            w.g[i][s] = __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 2);   // nt
            w.u[i][s] = __builtin_amdgcn_raw_buffer_load_b128(rs, o + 2 * (int)I, 0, 2);
        }
}

__device__ __forceinline__ void stage_a1_pairs(float* R2, const A1Words& w, int lane) {
    const int c8 = lane & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int row = (lane >> 3) + 8 * i, col = 64 * s + 8 * c8;
            float x[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {      // word k: columns 2k, 2k+1
                const uint32_t gw = w.g[i][s][k], uw = w.u[i][s][k];
                x[2 * k] = __uint_as_float((gw & 0xffffu) | (uw << 16));
                x[2 * k + 1] = __uint_as_float((gw >> 16) | (uw & 0xffff0000u));
            }
            store_row8(R2, row, col, x);
        }
}

// (gate, up) of staged pair x
__device__ __forceinline__ float pair_gate(float x) { return lo_bf16(__float_as_uint(x)); }
__device__ __forceinline__ float pair_up(float x) { return hi_bf16(__float_as_uint(x)); }

// SwiGLU backward of row slice fi: staged columns are dA2 for j = n0 + wn*128
// + col.  Writes dA1 (bf16, or rowwise + columnwise MXFP8) and the row's
// probability-gradient partial over these 128 columns into red.
template <int DT>
__device__ __forceinline__ void swiglu_bwd_rows(const EpiCtx& c, float* R, float* R2,
                                                float* red, const f32x16& f0, const f32x16& f1,
                                                const f32x16& f2, const f32x16& f3, int fi,
                                                uint32_t& amx, A1Words& w) {
    const GemmArgs& g = c.g;
    const Tile& tl = c.tl;
    const int lane = c.lane;
    const int64_t I = g.I;
    stage_fragments(R, f0, f1, f2, f3, lane);
    wave_lds_sync();
    const int frow0 = tl.m0 + c.wm * 128 + fi * 32;
    const int valid = min(32, tl.rows_e - frow0);
    const int jw = tl.n0 + c.wn * 128;                      // first column of the wave
    const bool slab = jw < I;                              // I % 128 == 0: all or nothing
    const int row = lane >> 1, h = lane & 1;
    if (slab && valid > 0) stage_a1_pairs(R2, w, lane);
    if (fi > 0) load_a1(g, tl, c.wm, c.wn, fi - 1, lane, w);   // the next slice's, in flight
    wave_lds_sync();
    float part = 0.f;
    {
        // phase 1, 8 values at a time: dg replaces the staged dA2 in R, du
        // replaces the staged gate/up pairs in R2 (rows past the expert stay
        // zero for the column blocks).  MXFP8: each 32-column block of dg and
        // of du is also held in registers and quantized rowwise right away,
        // its 32 codes stored as one 32-byte run of the row-pair layout.
        const bool live = slab && row < valid;
        const float p = live ? c.pr[fi] : 0.f;
        const int64_t rp = tl.pbase + frow0 + row;           // expert-padded row
        const int64_t ps = p2_stride(2 * I);
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const int cb = 64 * h + 32 * blk;
            float gq[32], uq[32];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                float d[8], pr8[8], dg[8], du[8];
                load_row8(R, row, cb + 8 * b, d);
                load_row8(R2, row, cb + 8 * b, pr8);     // read before du takes the slots
                if (live) {
                    float gt[8], up[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        gt[i] = pair_gate(pr8[i]);
                        up[i] = pair_up(pr8[i]);
                    }
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        float sg = sigmoid_f(gt[i]);
                        float sl = gt[i] * sg;
                        float dp = d[i] * p;
                        dg[i] = dp * up[i] * sg * (1.f + gt[i] * (1.f - sg));
                        du[i] = dp * sl;
                        part += d[i] * sl * up[i];
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) dg[i] = du[i] = 0.f;
                }
                store_row8(R, row, cb + 8 * b, dg);
                store_row8(R2, row, cb + 8 * b, du);
                if (DT == DT_MX)
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        gq[8 * b + i] = dg[i];
                        uq[8 * b + i] = du[i];
                    }
            }
            if (DT == DT_MX && live) {
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const int64_t j = (s2 ? I : 0) + jw + cb;   // first column of the block
                    u32x4 c0, c1;
                    const uint32_t S = quant32(s2 ? uq : gq, c0, c1);
                    u32x4* o = (u32x4*)(g.q_row + p2_off(rp, j, ps));
                    o[0] = c0;
                    o[1] = c1;
                    g.q_row_s[(j / 32) * g.rows_pad + rp] = (uint8_t)S;
                }
            }
        }
    }
    if (DT != DT_MX) {
        // bf16 dA1 = [dg, du] in whole 128-byte lines: 8 lanes per line of a
        // row, 8 rows per instruction, streamed past L2
        wave_lds_sync();
        if (slab) {
            const int c8 = lane & 7;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = (lane >> 3) + 8 * i;
                if (r < valid) {
                    const int64_t gr = tl.row0 + frow0 + r;
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const int col = 64 * s + 8 * c8;
                        float x[8];
                        load_row8(R, r, col, x);
                        const u32x4 pg = pack8_bf16(x);
                        load_row8(R2, r, col, x);
                        const u32x4 pu = pack8_bf16(x);
                        __builtin_nontemporal_store(pg, (u32x4*)(g.act + gr * 2 * I + jw + col));
                        __builtin_nontemporal_store(pu, (u32x4*)(g.act + gr * 2 * I + I + jw + col));
                        if (DT == DT_FP8)   // the tensor maximum of the cast that follows
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                amx = max_abs_bf16x2(max_abs_bf16x2(amx, pg[q]), pu[q]);
                    }
                }
            }
        }
    } else {
        // columnwise MXFP8 (lane = column, its 32 rows; phase 1 staged zeros
        // for the rows past the expert)
        wave_lds_sync();
        if (slab && valid > 0) {
#pragma unroll 1
            for (int t = 0; t < 4; ++t) {
                const int col = lane + 64 * t;              // 0..127 dg, 128..255 du
                const int cc = col & 127;
                const int64_t j = (col < 128 ? 0 : I) + jw + cc;
                col_quant(col < 128 ? R : R2, cc,
                          g.q_col + tl.pbase64 * 2 * I + p2_off(j, frow0, 2 * tl.pad64_e),
                          g.q_col_s + tl.pbase / 32 * 2 * I + (frow0 / 32) * 2 * I + j);
            }
        }
    }
    part += __shfl_xor(part, 1);
    if (h == 0) red[c.wn * kGemmBM + c.wm * 128 + fi * 32 + row] = part;
    wave_lds_sync();
}

// The lane index recomputed from the execution mask (all lanes are active)
// and passed through an empty asm, for the epilogues: it then depends on
// nothing computed before the K loop, so neither the work-item id nor
// addresses built on it are kept live (and spilled) through the loop.
__device__ __forceinline__ int lane_after_loop() {
    int l = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    asm volatile("" : "+v"(l));
    return l;
}

// Workgroup maximum of the lanes' values into part[blockIdx.x] (scratch: 4
// words of LDS no longer in use).
__device__ __forceinline__ void amax_to_part(uint32_t v, uint32_t* scratch, uint32_t* part) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) scratch[wave] = v;
    __syncthreads();
    if (threadIdx.x == 0)
        part[blockIdx.x] = max(max(scratch[0], scratch[1]), max(scratch[2], scratch[3]));
}

// ---------------------------------------------------------------- the kernel
template <int DT, int LA, int LB, int GRP, int EPI, int USE>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_kernel(GemmArgs g, int ntn, int mtm) {
    // One LDS array per pipeline stage: with the K loop unrolled by the stage
    // count every access names its stage statically, which lets the compiler
    // see that the DMA into one stage does not alias the reads of another
    // (otherwise it waits for all DMA before every LDS read).
    __shared__ __attribute__((aligned(16))) uint8_t lds0[kStageB];
    __shared__ __attribute__((aligned(16))) uint8_t lds1[kStageB];
    __shared__ __attribute__((aligned(16))) uint8_t lds2[kStageB];
    __shared__ __attribute__((aligned(16))) uint8_t lds3[kStageB];
    __shared__ __attribute__((aligned(16))) uint8_t ssc[kStages][2][2][kGemmBM];   // MXFP8 scales
    __shared__ float red[2 * kGemmBM];                  // probability-gradient row partials
    __shared__ int sched[384];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);      // uniform
    const int wm = wave >> 1, wn = wave & 1;

    // XCD-aware remap: dispatch is round-robin over 8 XCDs; hand XCD x the
    // contiguous logical range [x*G/8, (x+1)*G/8).
    const int G8 = gridDim.x >> 3;
    const int t = (blockIdx.x & 7) * G8 + (blockIdx.x >> 3);

    constexpr bool kAmax = DT == DT_FP8 && (EPI == EPI_SWIGLU_FWD || EPI == EPI_SWIGLU_BWD);
    Tile tl;
    if (!decode_tile<GRP>(g, ntn, mtm, t, sched, tl)) {
        if (kAmax && tid == 0) g.amax_part[blockIdx.x] = 0;
        return;
    }

    // ---- operand descriptors
    constexpr int kElemB = DT == DT_BF16 ? 2 : 1;
    KOp ka{}, kb{};
    MNOp ma{}, mb{};
    int kext;                          // K extent in elements
    const uint8_t* sbase_a = nullptr;  // MXFP8 scale arrays (block-major), the offsets of
    const uint8_t* sbase_b = nullptr;  // this lane's 4-row group and the block-row lengths
    uint32_t soff_a = 0, soff_b = 0, sld_a = 0, sld_b = 0;
    const int r4 = (lane & 63) * 4;    // first of the 4 tile rows whose scales this lane loads
    int nblk = 0;
    constexpr bool kP2 = DT != DT_BF16;    // 8-bit operands: row-pair layout
    if (GRP == G_M) {
        kext = g.K;
        if (kP2) {
            // the expert's rows start at its padded row base (a multiple of
            // 32), so the tile's first row starts a row pair
            const int64_t rp = tl.pbase + tl.m0;
            ka.stride = p2_stride(g.K);
            ka.base = (const uint8_t*)g.a + (rp >> 1) * ka.stride;
            ka.rows_valid = tl.rows_e - tl.m0;
        } else {
            ka.base = (const uint8_t*)g.a + (tl.row0 + tl.m0) * g.lda * kElemB;
            ka.stride = g.lda * kElemB;
            ka.rows_valid = (int)(g.rows - (tl.row0 + tl.m0));
        }
        ka.row_first = 0;
        ka.kbytes = g.K * kElemB;
        if (LB == L_KMAJ) {
            kb.base = (const uint8_t*)g.b.p[tl.e];
            kb.stride = kP2 ? p2_stride(g.K) : g.ldb * kElemB;
            kb.row_first = tl.n0;
            kb.rows_valid = EPI == EPI_SWIGLU_FWD ? 2 * g.I : g.N;
            kb.kbytes = g.K * kElemB;
            kb.pair_I = EPI == EPI_SWIGLU_FWD ? g.I : 0;
            kb.j0 = tl.n_tile * (kGemmBN / 2);
        } else {
            mb.base = (const uint8_t*)g.b.p[tl.e] + (int64_t)tl.n0 * 2;
            mb.stride = g.ldb * 2;
            mb.k_valid = g.K;
            mb.mn_valid = g.N - tl.n0;
        }
        if (DT != DT_BF16) {
            nblk = g.K / 32;
            sbase_a = g.a_scale;
            soff_a = r4 < ka.rows_valid ? (uint32_t)(tl.pbase + tl.m0 + r4) : kOob;
            sld_a = (uint32_t)g.rows_pad;
            sbase_b = (const uint8_t*)g.b_scale.p[tl.e];
            soff_b = (kb.pair_I > 0 || kb.row_first + r4 < kb.rows_valid)
                         ? (uint32_t)kop_row(kb, r4) : kOob;
            sld_b = (uint32_t)kb.rows_valid;
        }
    } else {
        kext = DT != DT_BF16 ? tl.pad_e : tl.rows_e;
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
            // grouped columnwise operands in the row-pair layout: the group of
            // expert e at C * pbase64_e, its rows (the columns of the
            // activation) 2p, 2p+1 sharing lines of its 64-padded K extent
            const int64_t ps = (int64_t)tl.pad64_e * 2;
            ka.base = (const uint8_t*)g.a + tl.pbase64 * g.M + (tl.m0 >> 1) * ps;
            ka.stride = ps;
            ka.row_first = 0;
            ka.rows_valid = g.M - tl.m0;
            ka.kbytes = tl.pad_e;
            kb.base = (const uint8_t*)g.b.p[0] + tl.pbase64 * g.N + (tl.n0 >> 1) * ps;
            kb.stride = ps;
            kb.row_first = 0;
            kb.rows_valid = g.N - tl.n0;
            kb.kbytes = tl.pad_e;
            nblk = tl.pad_e / 32;
            sbase_a = g.a_scale + tl.pbase / 32 * g.M;
            soff_a = tl.m0 + r4 < g.M ? (uint32_t)(tl.m0 + r4) : kOob;
            sld_a = (uint32_t)g.M;
            sbase_b = (const uint8_t*)g.b_scale.p[0] + tl.pbase / 32 * g.N;
            soff_b = tl.n0 + r4 < g.N ? (uint32_t)(tl.n0 + r4) : kOob;
            sld_b = (uint32_t)g.N;
        }
    }
    constexpr int kStepElems = DT == DT_BF16 ? 32 : 64;   // K per stage (64 bytes per row)
    const int nk = (kext + kStepElems - 1) / kStepElems;

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // One batch of loads per K step, always issued in the same order and
    // number (DMA A: 4, DMA B: 4, MXFP8 scales: 1) so that "wait until at
    // most two batches are outstanding" is a fixed vmcnt.  Steps past the end
    // read zeros into stages that are never consumed.
    constexpr int kBatch = 8 + (DT != DT_BF16 ? 1 : 0);
    constexpr int kWait2 = 2 * kBatch;                           // vmcnt(2 batches)
    // (M/N-contiguous operands build their buffer resource per K step)
    const i32x4 rs_a = make_rsrc(LA == L_KMAJ ? (const void*)ka.base : nullptr);
    const i32x4 rs_b = make_rsrc(LB == L_KMAJ ? (const void*)kb.base : nullptr);
    const i32x4 rs_sa = make_rsrc(sbase_a), rs_sb = make_rsrc(sbase_b);

    auto stage_ptr = [&](auto S) -> uint8_t* {
        constexpr int st = decltype(S)::value % kStages;
        return st == 0 ? lds0 : st == 1 ? lds1 : st == 2 ? lds2 : lds3;
    };
    // issue the loads of K step kt into stage S
    auto issue = [&](auto S, int kt) {
        constexpr int st = decltype(S)::value % kStages;
        uint8_t* base = stage_ptr(S);
        if (LA == L_KMAJ) dma_kop<kP2>(ka, rs_a, kt * kRowB, base);
        else dma_mnop(ma, kt * 32, base);
        if (LB == L_KMAJ) dma_kop<kP2>(kb, rs_b, kt * kRowB, base + kTileB);
        else dma_mnop(mb, kt * 32, base + kTileB);
        if (DT != DT_BF16)
            dma_scales(rs_sa, rs_sb, soff_a, soff_b, sld_a, sld_b, kt, nblk, ssc[st]);
    };

    const int fr = lane & 31, hi = lane >> 5;
    // Per-lane byte offsets of the K-contiguous fragment reads inside a stage.
    // Fragment f covers tile rows base + 32 f + fr; 32 f leaves the chunk
    // swizzle (row >> 2) & 3 = (fr >> 2) & 3 unchanged, so 16-byte chunk c of
    // fragment f lies at o_c + 32 f * kRowB: two offsets per operand (chunks
    // hi and 2 + hi), every read of a stage an immediate offset from them.
    const int oA0 = lds_off(wm * 128 + fr, hi), oA2 = lds_off(wm * 128 + fr, 2 + hi);
    const int oB0 = lds_off(wn * 128 + fr, hi), oB2 = lds_off(wn * 128 + fr, 2 + hi);
    constexpr int kFragB = 32 * kRowB;
    // The operand fragments of one K step, held in registers.  Two sets
    // alternate: while the MFMAs consume step k's set, the LDS reads of step
    // k+1 fill the other, so LDS latency is hidden behind matrix work instead
    // of stalling the wave before each group of MFMAs.
    struct FragsMX { i32x8 a[4]; i32x8 b[4]; uint32_t sa[4]; uint32_t sb[4]; };
    struct FragsBF { bf16x8_t a[2][4]; bf16x8_t b[2][4]; };
    using Frags = std::conditional_t<DT == DT_BF16, FragsBF, FragsMX>;

    // LDS -> registers: every fragment of the K step held in stage S
    auto load = [&](auto S, Frags& F) {
        constexpr int st = decltype(S)::value % kStages;
        const uint8_t* A = stage_ptr(S);
        const uint8_t* B = A + kTileB;
        if constexpr (DT == DT_BF16) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
#pragma unroll
                for (int fj = 0; fj < 4; ++fj) {
                    if (LB == L_KMAJ)
                        F.b[s][fj] = *(const bf16x8_t*)(B + (s ? oB2 : oB0) + fj * kFragB);
                    else
                        F.b[s][fj] = mn_frag(B, s, wn * 128 + fj * 32);
                }
#pragma unroll
                for (int fi = 0; fi < 4; ++fi) {
                    if (LA == L_KMAJ)
                        F.a[s][fi] = *(const bf16x8_t*)(A + (s ? oA2 : oA0) + fi * kFragB);
                    else
                        F.a[s][fi] = mn_frag(A, s, wm * 128 + fi * 32);
                }
            }
        } else {
            // Operand layout of the scaled 32x32x64 MFMA: lane (row r, half h)
            // holds K [16h, 16h+16) and [32+16h, 32+16h+16) of the 64-K step;
            // the E8M0 scale of K-block 0 of row r is taken from lane r, that
            // of block 1 from lane r+32 (byte h of the staged scale pair).
#pragma unroll
            for (int fj = 0; fj < 4; ++fj) {
                int row = wn * 128 + fj * 32 + fr;
                u32x4 lo = *(const u32x4*)(B + oB0 + fj * kFragB);
                u32x4 up = *(const u32x4*)(B + oB2 + fj * kFragB);
                F.b[fj] = (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                  (int)up[0], (int)up[1], (int)up[2], (int)up[3]};
                F.sb[fj] = ssc[st][1][hi][row];          // byte -> low 8 bits
            }
#pragma unroll
            for (int fi = 0; fi < 4; ++fi) {
                int row = wm * 128 + fi * 32 + fr;
                u32x4 lo = *(const u32x4*)(A + oA0 + fi * kFragB);
                u32x4 up = *(const u32x4*)(A + oA2 + fi * kFragB);
                F.a[fi] = (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                  (int)up[0], (int)up[1], (int)up[2], (int)up[3]};
                F.sa[fi] = ssc[st][0][hi][row];
            }
        }
    };
    // the MFMAs of fragment rows [FI0, FI1) of one K step; each accumulator
    // takes the step's K values in increasing order whatever the split
    auto mma = [&](auto FI0, auto FI1, const Frags& F) {
        constexpr int f0 = decltype(FI0)::value, f1 = decltype(FI1)::value;
#pragma unroll
        for (int fi = f0; fi < f1; ++fi) {
            if constexpr (DT == DT_BF16) {
#pragma unroll
                for (int s = 0; s < 2; ++s)
#pragma unroll
                    for (int fj = 0; fj < 4; ++fj)
                        acc[fi][fj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            F.a[s][fi], F.b[s][fj], acc[fi][fj], 0, 0, 0);
            } else {
#pragma unroll
                for (int fj = 0; fj < 4; ++fj)
                    acc[fi][fj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        F.a[fi], F.b[fj], acc[fi][fj], 0, 0, 0, (int)F.sa[fi], 0, (int)F.sb[fj]);
            }
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using I4 = std::integral_constant<int, 4>;
    // fragment rows whose MFMAs run after the barrier, under the next step's
    // LDS reads: 8 of the 16 scaled MFMAs, 8 of the 32 bf16 ones (measured
    // best; the bf16 step has 16 fragment reads against the 8-bit step's 24)
    constexpr int kTailRows = DT == DT_BF16 ? 1 : 2;
    using ISplit = std::integral_constant<int, 4 - kTailRows>;
    // One K step kt whose fragments are in Fc (read from stage S): prefetch
    // step kt+3 into stage S+3 (whose reads all finished before the previous
    // barrier), run most MFMAs, wait until batch kt+1 has landed in every
    // wave, read its fragments into Fn, and run the remaining MFMAs.
    Frags F0, F1;
    auto step = [&](auto S, int kt, Frags& Fc, Frags& Fn) {
        constexpr int st = decltype(S)::value;
        // (scheduling barriers keep the compiler from sinking the reads of Fn
        // to their first use, which would stall the next step's MFMAs on LDS)
        issue(std::integral_constant<int, (st + 3) % kStages>{}, kt + 3);
        mma(I0{}, ISplit{}, Fc);
        __builtin_amdgcn_sched_barrier(0);
        pipe_barrier<kWait2>();                                  // batch kt+1 has landed
        __builtin_amdgcn_sched_barrier(0);
        load(std::integral_constant<int, (st + 1) % kStages>{}, Fn);
        mma(ISplit{}, I4{}, Fc);
        // The next step's LDS reads spread between the MFMAs after the
        // barrier, the first MFMA ahead of them: the matrix pipe stays busy
        // while the reads trickle into LDS, and every read has several MFMAs
        // to land behind.  (Left to itself the compiler put all reads after
        // the sixth MFMA, two MFMAs before their first use; all 24 reads up
        // front, ahead of the MFMAs, was slower still.)
        if constexpr (DT == DT_BF16) {
            // reads per step: 8 per K-contiguous operand, 16 (transposing
            // 8-byte reads) per M/N-contiguous one
            constexpr int kReads = (LA == L_KMAJ ? 8 : 16) + (LB == L_KMAJ ? 8 : 16);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x100, kReads / 8, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
            }
        } else {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
            for (int i = 0; i < 6; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    if (nk > 0) {
        issue(I0{}, 0);
        issue(I1{}, 1);
        issue(I2{}, 2);
    }
    pipe_barrier<kWait2>();                                      // batch 0 has landed
    load(I0{}, F0);
    __builtin_amdgcn_sched_barrier(0);
    // whole groups of four steps, then the rest: a conditional step inside
    // the loop body makes the register allocator shuttle accumulators
    // between register files on every iteration
    int kt = 0;
    for (; kt + kStages <= nk; kt += kStages) {
        step(I0{}, kt, F0, F1);
        step(I1{}, kt + 1, F1, F0);
        step(I2{}, kt + 2, F0, F1);
        step(I3{}, kt + 3, F1, F0);
    }
    if (kt < nk) step(I0{}, kt, F0, F1);
    if (kt + 1 < nk) step(I1{}, kt + 1, F1, F0);
    if (kt + 2 < nk) step(I2{}, kt + 2, F0, F1);
    // the look-ahead batches past the end still write LDS: drain them before
    // the epilogue reuses it
    pipe_barrier<0>();

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
        // Each 32-row slice of the wave's 128 x 128 result goes through the
        // wave's own LDS region (the pipeline has drained), converted to bf16
        // row pairs on the way in, so that a lane stores 8 neighbouring
        // columns of two rows as two 16-byte writes (4 rows x 256 bytes per
        // instruction) instead of 2-byte writes column by column.  (The
        // SwiGLU epilogues keep ordinary stores: their instructions write
        // 16-byte pieces of a line, which L2 must merge.)
        float* R = (float*)(wave == 0 ? lds0 : wave == 1 ? lds1 : wave == 2 ? lds2 : lds3);
        const int ln = lane_after_loop();
        const int c8 = (ln & 15) * 8;
        const int gcol = wn * 128 + c8;             // N is a multiple of 8: all or nothing
        const int r0 = ln >> 4;
        // the lane's byte offset from its instruction's first row: the same
        // for every store, whose row base is uniform (scalar arithmetic)
        const uint32_t loff = (uint32_t)(r0 * ldc + gcol) * 2u;
        const bool cok = gcol < col_lim;
        // (slices in reverse order: the compiler then keeps every accumulator
        // in place through the epilogue instead of parking one fragment in
        // scratch memory)
        // slices staged as bf16 row pairs (half the LDS bytes of fp32): a
        // lane reads 8 columns of one row pair (two 16-byte reads) and
        // stores them as two 16-byte row pieces
        uint32_t* P = (uint32_t*)R;
        // byte offsets of the lane's two rows (2 r0 and 2 r0 + 1 of its
        // instruction's first row pair) at its 8 columns
        const uint32_t lo_off = (uint32_t)(2 * r0 * ldc + gcol) * 2u;
        const uint32_t hi_off = lo_off + (uint32_t)ldc * 2u;
#pragma unroll
        for (int fr = 0; fr < 4; ++fr) {
            const int fi = 3 - fr;
            stage_pairs_bf16(P, acc[fi][0], acc[fi][1], acc[fi][2], acc[fi][3], ln);
            wave_lds_sync();
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int p = r0 + 4 * i;                          // row pair of the slice
                const int urow = wm * 128 + fi * 32 + 8 * i;       // uniform
                const u32x4 d0 = *(const u32x4*)(P + p * 128 + c8);
                const u32x4 d1 = *(const u32x4*)(P + p * 128 + c8 + 4);
                u32x4 lo, hi2;
                lo[0] = __builtin_amdgcn_perm(d0[1], d0[0], 0x05040100u);
                lo[1] = __builtin_amdgcn_perm(d0[3], d0[2], 0x05040100u);
                lo[2] = __builtin_amdgcn_perm(d1[1], d1[0], 0x05040100u);
                lo[3] = __builtin_amdgcn_perm(d1[3], d1[2], 0x05040100u);
                hi2[0] = __builtin_amdgcn_perm(d0[1], d0[0], 0x07060302u);
                hi2[1] = __builtin_amdgcn_perm(d0[3], d0[2], 0x07060302u);
                hi2[2] = __builtin_amdgcn_perm(d1[1], d1[0], 0x07060302u);
                hi2[3] = __builtin_amdgcn_perm(d1[3], d1[2], 0x07060302u);
                const char* rb = (const char*)C + (int64_t)urow * ldc * 2;
                // streaming stores: the output is not read again by this
                // kernel, so it should not evict the operands from L2
                if (cok && 2 * r0 < row_lim - urow)
                    __builtin_nontemporal_store(lo, (u32x4*)(rb + lo_off));
                if (cok && 2 * r0 + 1 < row_lim - urow)
                    __builtin_nontemporal_store(hi2, (u32x4*)(rb + hi_off));
            }
            wave_lds_sync();
        }
        return;
    }

    // the routing probability of the lane's row in each 32-row slice, loaded
    // once for the whole epilogue (rows past the expert are never used)
    const int ln = lane_after_loop();
    A1Words a1w;
    if (EPI == EPI_SWIGLU_BWD) load_a1(g, tl, wm, wn, 3, ln, a1w);   // the first slice's saved A1
    float pr[4] = {0.f, 0.f, 0.f, 0.f};
    if (EPI == EPI_SWIGLU_FWD || EPI == EPI_SWIGLU_BWD) {
#pragma unroll
        for (int fi = 0; fi < 4; ++fi) {
            const int frow = tl.m0 + wm * 128 + fi * 32 + (ln >> 1);
            if (frow < tl.rows_e) pr[fi] = g.prob[tl.row0 + frow];
        }
    }

    if (EPI == EPI_SWIGLU_FWD) {
        EpiCtx c{g, tl, wm, wn, ntn, {pr[0], pr[1], pr[2], pr[3]}, ln};
        float* R = (float*)(wave == 0 ? lds0 : wave == 1 ? lds1 : wave == 2 ? lds2 : lds3);
        uint32_t amx = 0;
        // (slices in reverse order, as in the plain-store epilogue: no
        // accumulator fragment is parked in scratch memory)
        swiglu_fwd_rows<DT>(c, R, acc[3][0], acc[3][1], acc[3][2], acc[3][3], 3, amx);
        swiglu_fwd_rows<DT>(c, R, acc[2][0], acc[2][1], acc[2][2], acc[2][3], 2, amx);
        swiglu_fwd_rows<DT>(c, R, acc[1][0], acc[1][1], acc[1][2], acc[1][3], 1, amx);
        swiglu_fwd_rows<DT>(c, R, acc[0][0], acc[0][1], acc[0][2], acc[0][3], 0, amx);
        if (kAmax) amax_to_part(amx, (uint32_t*)sched, g.amax_part);
        return;
    }

    if (EPI == EPI_SWIGLU_BWD) {
        EpiCtx c{g, tl, wm, wn, ntn, {pr[0], pr[1], pr[2], pr[3]}, ln};
        float* R = (float*)(wave == 0 ? lds0 : wave == 1 ? lds1 : wave == 2 ? lds2 : lds3);
        float* R2 = R + 32 * 128;
        uint32_t amx = 0;
        // (slices in reverse order: no accumulator fragment parked in scratch)
        swiglu_bwd_rows<DT>(c, R, R2, red, acc[3][0], acc[3][1], acc[3][2], acc[3][3], 3, amx, a1w);
        swiglu_bwd_rows<DT>(c, R, R2, red, acc[2][0], acc[2][1], acc[2][2], acc[2][3], 2, amx, a1w);
        swiglu_bwd_rows<DT>(c, R, R2, red, acc[1][0], acc[1][1], acc[1][2], acc[1][3], 1, amx, a1w);
        swiglu_bwd_rows<DT>(c, R, R2, red, acc[0][0], acc[0][1], acc[0][2], acc[0][3], 0, amx, a1w);
        if (kAmax) amax_to_part(amx, (uint32_t*)sched, g.amax_part);
        __syncthreads();                    // red holds both column halves' partials
        const int t = wave * 64 + ln;
        if (tl.m0 + t < tl.rows_e)
            g.dprob_part[(tl.row0 + tl.m0 + t) * (int64_t)ntn + tl.n_tile] =
                red[t] + red[kGemmBM + t];
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

int64_t gemm_slots(int grp, int epi, int64_t rows, int E, int M, int N, int I) {
    const int ntn = gemm_n_tiles(epi, N, I);
    int64_t tiles;
    if (grp == G_M)   // upper bound of sum_e ceil(M_e / BM)
        tiles = (rows + (int64_t)E * (kGemmBM - 1)) / kGemmBM * ntn;
    else
        tiles = (int64_t)E * ((M + kGemmBM - 1) / kGemmBM) * ntn;
    return (tiles + 7) / 8 * 8;
}

int64_t padded_rows(int64_t rows, int E) { return ((rows + 31) / 32 + (E > 1 ? E : 1)) * 32; }

size_t grouped_p2_bytes(int64_t rows, int64_t C, int E) {
    // C columns of sum_e 64 ceil(M_e / 64) <= 64 (ceil(rows / 64) + E) K bytes
    return (size_t)C * 64 * (size_t)((rows + 63) / 64 + (E > 1 ? E : 1));
}

template <int DT, int LA, int LB, int GRP, int EPI, int USE>
static hipError_t run(const GemmArgs& g, hipStream_t s) {
    const int ntn = gemm_n_tiles(EPI, g.N, g.I);
    const int mtm = GRP == G_M ? 0 : (g.M + kGemmBM - 1) / kGemmBM;
    const int64_t grid = gemm_slots(GRP, EPI, g.rows, g.E, g.M, g.N, g.I);
    if (grid == 0) return hipSuccess;
    TraceScope ts(g.name ? g.name : "gemm", s);
    gemm_kernel<DT, LA, LB, GRP, EPI, USE><<<(unsigned)grid, kGemmThreads, 0, s>>>(g, ntn, mtm);
    return hipGetLastError();
}

hipError_t launch_gemm(int dtype, int use, const GemmArgs& g, hipStream_t s) {
    // FP8 (per-tensor scales, stored as uniform block scales) differs from
    // MXFP8 only where an epilogue produces the next GEMM's operand: there it
    // writes bf16, cast once the tensor's amax is known
    if (dtype == DT_FP8 && use != U_GATEUP_FWD && use != U_DOWN_DGRAD) dtype = DT_MX;
#define MOE_GEMM_CASE(DT, USE, LA, LB, GRP, EPI) \
    if (dtype == DT && use == USE) return run<DT, LA, LB, GRP, EPI, USE>(g, s);
    // bf16: the backward reads W1, W2 and both weight-gradient operands in
    // their natural (M/N-contiguous) layout
    MOE_GEMM_CASE(DT_BF16, U_GATEUP_FWD, L_KMAJ, L_KMAJ, G_M, EPI_SWIGLU_FWD)
    MOE_GEMM_CASE(DT_BF16, U_DOWN_FWD, L_KMAJ, L_KMAJ, G_M, EPI_STORE)
    MOE_GEMM_CASE(DT_BF16, U_DOWN_DGRAD, L_KMAJ, L_MNMAJ, G_M, EPI_SWIGLU_BWD)
    MOE_GEMM_CASE(DT_BF16, U_DOWN_WGRAD, L_MNMAJ, L_MNMAJ, G_K, EPI_STORE)
    MOE_GEMM_CASE(DT_BF16, U_GATEUP_DGRAD, L_KMAJ, L_MNMAJ, G_M, EPI_STORE)
    MOE_GEMM_CASE(DT_BF16, U_GATEUP_WGRAD, L_MNMAJ, L_MNMAJ, G_K, EPI_STORE)
    // mxfp8: every operand is quantized along its GEMM's K, K-contiguous
    MOE_GEMM_CASE(DT_MX, U_GATEUP_FWD, L_KMAJ, L_KMAJ, G_M, EPI_SWIGLU_FWD)
    MOE_GEMM_CASE(DT_MX, U_DOWN_FWD, L_KMAJ, L_KMAJ, G_M, EPI_STORE)
    MOE_GEMM_CASE(DT_MX, U_DOWN_DGRAD, L_KMAJ, L_KMAJ, G_M, EPI_SWIGLU_BWD)
    MOE_GEMM_CASE(DT_MX, U_DOWN_WGRAD, L_KMAJ, L_KMAJ, G_K, EPI_STORE)
    MOE_GEMM_CASE(DT_MX, U_GATEUP_DGRAD, L_KMAJ, L_KMAJ, G_M, EPI_STORE)
    MOE_GEMM_CASE(DT_MX, U_GATEUP_WGRAD, L_KMAJ, L_KMAJ, G_K, EPI_STORE)
    MOE_GEMM_CASE(DT_FP8, U_GATEUP_FWD, L_KMAJ, L_KMAJ, G_M, EPI_SWIGLU_FWD)
    MOE_GEMM_CASE(DT_FP8, U_DOWN_DGRAD, L_KMAJ, L_KMAJ, G_M, EPI_SWIGLU_BWD)
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
