// Internal launcher interface between the C ABI (capi.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxExperts = 64;
constexpr int kMaxTopK = 64;

typedef uint16_t bf16_t;

// A table of per-matrix (per-expert) device pointers, passed by value in the
// kernel arguments (64 x 8 B = 512 B).
struct MatTable {
    const void* p[kMaxExperts];
};

// ---- routing / permutation
size_t route_workspace_bytes(int64_t T, int E, int k);
// The no-allocation routing scratch: a static device array of this many bytes
// per device; route_scratch() returns its device address on the current
// device (taken once per device).
constexpr size_t kRouteScratchBytes = (size_t)8 << 20;
constexpr int kMaxDevices = 64;
hipError_t route_scratch(void** ptr);
hipError_t launch_route(const float* logits, int T, int E, int k, uint32_t flags,
                        int32_t* topk_expert, float* topk_prob, int32_t* split_sizes,
                        int32_t* expert_offsets, int32_t* dest_row, int32_t* src_token,
                        void* ws, hipStream_t s);
hipError_t launch_route_bwd(const float* topk_prob, const float* dprob_perm,
                            const int32_t* dest_row, const int32_t* topk_expert,
                            const float* logits, int T, int E, int k, uint32_t flags,
                            float* dlogits, hipStream_t s);
hipError_t launch_permute(const bf16_t* x, int T, int H, int k, const int32_t* dest_row,
                          const float* topk_prob, bf16_t* xp, float* prob_perm, hipStream_t s);
hipError_t launch_unpermute(const bf16_t* yp, int T, int H, int k, const int32_t* dest_row,
                            const float* topk_prob, bf16_t* y, hipStream_t s);

// ---- router linear layer
size_t router_bwd_workspace_bytes(int64_t T, int H, int E);
hipError_t launch_check_routing(const int32_t* split, int E, int64_t rows,
                                const int32_t* dest_row, const int32_t* src_token,
                                const int32_t* topk_expert, int64_t T, int k, int32_t* status,
                                hipStream_t s);
hipError_t launch_router_logits(const bf16_t* x, const bf16_t* w, int T, int H, int E,
                                float* logits, hipStream_t s);
hipError_t launch_router_bwd(const float* dlogits, const bf16_t* x, const bf16_t* w, int T,
                             int H, int E, int k, const int32_t* dest_row, const bf16_t* dxp,
                             bf16_t* dx, bf16_t* dw, void* ws, hipStream_t s);

// ---- MXFP8
int64_t colwise_block_bound(int64_t rows, int ngroups);
// scales_t: store the E8M0 scales block-major ([K/32][rows] for rowwise,
// [P_g/32][cols] per group for grouped columnwise), the layout the grouped
// GEMM reads with one coalesced load per K step; false = the public layout.
// Rowwise (rcodes given), grouped columnwise (ccodes given) or both, from one
// read of each matrix.
// p2_rows_pad > 0: the GEMM operand layouts (row-pair layout, common.hpp):
// row codes at expert-padded rows (groups from their 32-padded row bases),
// block-major row scales [cols/32][p2_rows_pad] (rscales_t required); grouped
// columnwise codes in the row-pair layout of [cols, 64-padded group rows] per
// group at cols * (sum of the earlier groups' 64-padded sizes), scales as in
// the public layout (cscales_t: block-major).  0: the public layouts.
hipError_t launch_quant(const MatTable& src, int nmat, const int32_t* sizes, int ngroups,
                        int64_t rows, int64_t cols, const MatTable* rcodes,
                        const MatTable* rscales, bool rscales_t, const MatTable* ccodes,
                        const MatTable* cscales, bool cscales_t, hipStream_t s,
                        const char* name, const float* fixed_amax = nullptr,
                        int64_t p2_rows_pad = 0, const int32_t* gather = nullptr);
// Per-tensor FP8: fixed_amax (device, one float per matrix) replaces the block
// maxima, so every block of matrix m gets the scale of amax[m].
// gather (one matrix, both orientations): row r of the quantized matrix is
// row gather[r] of src, so a permutation of token rows and their
// quantization are one pass.
// amax[m] = max |x| over matrix m's n values (n a multiple of 8); ws holds
// amax_workspace_bytes(nmat) bytes.
size_t amax_workspace_bytes(int nmat);
hipError_t launch_amax(const MatTable& src, int nmat, int64_t n, void* ws, float* amax,
                       hipStream_t s, const char* name);
// amax over the rows of a gathered matrix: rows x cols values, row r being
// row gather[r] of x (cols a multiple of 8); ws as for launch_amax(.., 1, ..).
hipError_t launch_amax_gather(const bf16_t* x, const int32_t* gather, int64_t rows, int64_t cols,
                              void* ws, float* amax, hipStream_t s, const char* name);
// The final reduction alone, over per-workgroup partials written elsewhere
// (the FP8 SwiGLU GEMM epilogues): amax[0] = the largest of part[0..nparts).
hipError_t launch_amax_final(const uint32_t* part, int nparts, float* amax, hipStream_t s,
                             const char* name);
hipError_t launch_quant_rows(const MatTable& src, const MatTable& codes, const MatTable& scales,
                             int nmat, int64_t rows, int64_t cols, hipStream_t s,
                             const char* name = "mx_quant_rows", bool scales_t = false,
                             int64_t p2_rows_pad = 0);
hipError_t launch_quant_cols(const MatTable& src, const MatTable& codes, const MatTable& scales,
                             int nmat, const int32_t* sizes, int ngroups, int64_t rows,
                             int64_t cols, hipStream_t s, const char* name = "mx_quant_cols",
                             bool scales_t = false, int64_t p2_rows_pad = 0);
// Bytes of an R x K 8-bit matrix in the row-pair layout.
inline size_t p2_bytes(int64_t R, int64_t K) {
    return (size_t)((R + 1) / 2) * (size_t)(((K + 63) / 64) * 128);
}
hipError_t launch_dequant_rows(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                               int64_t cols, bf16_t* out, hipStream_t s);
hipError_t launch_dequant_cols(const uint8_t* codes, const uint8_t* scales, const int32_t* sizes,
                               int ngroups, int64_t rows, int64_t cols, bf16_t* out,
                               hipStream_t s);

}  // namespace moe
