// Grouped GEMM launcher interface and the grouped-MLP orchestration.
#pragma once

#include "kernels.hpp"

namespace moe {

// Operand types: BF16; MXFP8 (E4M3 + E8M0 per 32 K-values, epilogues emit the
// next operand as MXFP8); FP8 (E4M3 with one scale per tensor, stored as
// uniform block scales, epilogues emit bf16 for a later per-tensor cast).
enum GemmDType { DT_BF16 = 0, DT_MX = 1, DT_FP8 = 2 };
enum GemmLayout { L_KMAJ = 0, L_MNMAJ = 1 };   // operand contiguous along K / along M or N
enum GemmGroup { G_M = 0, G_K = 1 };           // ragged rows (fwd, dgrad) / ragged K (wgrad)
enum GemmEpi { EPI_STORE = 0, EPI_SWIGLU_FWD = 1, EPI_SWIGLU_BWD = 2 };
// The six grouped GEMMs of the layer; each gets a kernel symbol of its own so
// that profiles attribute time per GEMM.
enum GemmUse {
    U_GATEUP_FWD = 0,    // xp W1^T, ScaledSwiGLU epilogue
    U_DOWN_FWD = 1,      // A2 W2^T
    U_DOWN_DGRAD = 2,    // dyp W2, SwiGLU-backward epilogue
    U_DOWN_WGRAD = 3,    // dyp^T A2 per expert
    U_GATEUP_DGRAD = 4,  // dA1 W1
    U_GATEUP_WGRAD = 5,  // dA1^T xp per expert
};

constexpr int kGemmBM = 256, kGemmBN = 256, kGemmThreads = 256;

// Arguments of one grouped GEMM C_e = A_e B_e^T over all experts e.
//
// G_M: expert e owns rows [row0_e, row0_e + M_e) of A and C (row-major, K
//      contiguous in A); B_e = b.p[e] is [N, K] (L_KMAJ) or [K, N] (L_MNMAJ).
// G_K: expert e owns rows [row0_e, row0_e + M_e) of two row-major matrices
//      and C_e (= c_tab.p[e], [M, N]) = A_rows^T B_rows, contracting over them
//      (bf16: both L_MNMAJ); MXFP8: both operands are the grouped columnwise
//      layouts, [M, P_e] and [N, P_e] at the group's offset (L_KMAJ).
// 8-bit operands (MXFP8, FP8) are in the row-pair layout (common.hpp): the
// G_M A operand in the expert-padded row order (rows_pad), the weights per
// expert, the grouped columnwise operands per group at C * (sum of the
// 64-padded sizes of earlier groups).  bf16 strides are in elements.
struct GemmArgs {
    const void* a;
    int64_t lda;
    const uint8_t* a_scale;
    int64_t lda_s;
    MatTable b;
    int64_t ldb;
    MatTable b_scale;
    int64_t ldb_s;
    const int32_t* split;
    int E;
    int64_t rows;       // total grouped rows
    int64_t rows_pad;   // 8-bit row operands (G_M A operand, epilogue row codes): rows
                        // in the expert-padded order (expert e from its 32-padded row
                        // base), the row stride of their block-major scales
    int M, N, K;        // G_M: N and K; G_K: M and N (K ragged)
    void* c;            // G_M output base (bf16)
    int64_t ldc;
    MatTable c_tab;     // G_K per-expert outputs (bf16 [M, N])
    // epilogue
    const float* prob;  // prob_perm [rows]
    bf16_t* a1;         // SWIGLU_FWD: out [rows, 2I]; SWIGLU_BWD: in
    bf16_t* act;        // SWIGLU_FWD: A2 bf16 [rows, I]; SWIGLU_BWD: dA1 bf16 [rows, 2I]
    uint8_t* q_row;     // MXFP8 rowwise codes of the epilogue output
    uint8_t* q_row_s;
    uint8_t* q_col;     // MXFP8 grouped columnwise codes of the epilogue output
    uint8_t* q_col_s;
    float* dprob_part;  // SWIGLU_BWD: [rows, n_tiles]
    uint32_t* amax_part;  // FP8 SwiGLU epilogues: per workgroup, the largest |bf16| bit
                          // pattern of the stored output ([gemm_slots(...)]; 0 if none)
    int I;              // intermediate size (SwiGLU epilogues)
    const char* name;   // kernel name in launch traces
};

hipError_t launch_gemm(int dtype, int use, const GemmArgs& g, hipStream_t s);
hipError_t launch_dprob_reduce(const float* part, int64_t rows, int ntiles, float* dprob,
                               hipStream_t s);
int gemm_n_tiles(int epi, int N, int I);
// Workgroups (tile slots, a multiple of 8) of one grouped GEMM launch.
int64_t gemm_slots(int grp, int epi, int64_t rows, int E, int M, int N, int I);
// Rows of the expert-padded order (an upper bound of sum_e 32 ceil(M_e / 32))
// and bytes of a grouped columnwise row-pair buffer of C columns.
int64_t padded_rows(int64_t rows, int E);
size_t grouped_p2_bytes(int64_t rows, int64_t C, int E);

size_t mlp_fwd_workspace_bytes(int64_t rows, int H, int I, int E, int precision);
int mlp_workspace_region(int op, int region, int64_t rows, int H, int I, int E, int precision,
                         size_t* offset, size_t* bytes);
size_t mlp_saved_bytes(int precision, int member, int64_t rows, int H, int I, int E);
size_t linear_fwd_workspace_bytes(int64_t rows, int N, int K, int E, int precision);
size_t linear_bwd_workspace_bytes(int64_t rows, int N, int K, int E, int precision);
size_t mlp_bwd_workspace_bytes(int64_t rows, int H, int I, int E, int precision);

}  // namespace moe
