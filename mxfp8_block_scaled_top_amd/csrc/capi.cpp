// C ABI of libmoe_mi355x: argument validation, workspace sizing and kernel
// launches.  Declarations and the contract of every call are in
// include/moe_mi355x.h.  No call allocates memory or synchronizes the host.
#include "moe_mi355x.h"

#include <hip/hip_runtime.h>
#include <string.h>

#include <mutex>

#include "kernels.hpp"
#include "mlp.hpp"

using namespace moe;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// gfx950 check, cached per device id.
int g_dev_ok[64];
std::once_flag g_dev_once[64];

bool device_ok() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
    std::call_once(g_dev_once[dev], [dev]() {
        hipDeviceProp_t prop;
        g_dev_ok[dev] = 0;
        if (hipGetDeviceProperties(&prop, dev) == hipSuccess)
            g_dev_ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
    });
    return g_dev_ok[dev] == 1;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "a required pointer is NULL";
        case MOE_ERR_SHAPE: return "a size is out of range or not a required multiple";
        case MOE_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_ERR_UNSUPPORTED: return "unsupported device (needs gfx950) or option";
        case MOE_ERR_HIP: return "HIP launch failed";
        case MOE_ERR_ARG: return "invalid enum or flag argument";
        default: return "unknown status";
    }
}

int moe_device_supported(void) { return device_ok() ? 1 : 0; }

size_t moe_workspace_bytes(int op, int64_t T, int H, int I, int E, int k, int precision) {
    if (T < 0 || E < 1 || E > kMaxExperts || k < 1 || k > E) return 0;
    switch (op) {
        case MOE_OP_ROUTE: return route_workspace_bytes(T, E, k);
        case MOE_OP_MLP_FWD: return mlp_fwd_workspace_bytes(T * k, H, I, E, precision);
        case MOE_OP_MLP_BWD: return mlp_bwd_workspace_bytes(T * k, H, I, E, precision);
        case MOE_OP_ROUTER_FWD: return route_workspace_bytes(T, E, k);
        case MOE_OP_ROUTER_BWD: return router_bwd_workspace_bytes(T, H, E);
        case MOE_OP_LINEAR_FWD: return k == 1 ? linear_fwd_workspace_bytes(T, I, H, E, precision) : 0;
        case MOE_OP_LINEAR_BWD: return k == 1 ? linear_bwd_workspace_bytes(T, I, H, E, precision) : 0;
        default: return 0;
    }
}

int moe_route(const float* logits, int64_t T, int E, int k, uint32_t flags, int32_t* topk_expert,
              float* topk_prob, int32_t* split_sizes, int32_t* expert_offsets, int32_t* dest_row,
              int32_t* src_token, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!split_sizes || !expert_offsets || !workspace) return MOE_ERR_NULL;
    if (T > 0 && (!logits || !topk_expert || !topk_prob || !dest_row || !src_token))
        return MOE_ERR_NULL;
    if (T < 0 || E < 1 || E > kMaxExperts || k < 1 || k > E || T * k > INT32_MAX)
        return MOE_ERR_SHAPE;
    if (flags > MOE_ROUTE_SOFTMAX_ALL) return MOE_ERR_ARG;
    if (workspace_bytes < route_workspace_bytes(T, E, k)) return MOE_ERR_WORKSPACE;
    if (!device_ok()) return MOE_ERR_UNSUPPORTED;
    return hip_status(launch_route(logits, (int)T, E, k, flags, topk_expert, topk_prob,
                                   split_sizes, expert_offsets, dest_row, src_token, workspace,
                                   stream));
}

int moe_route_noalloc(const float* logits, int64_t T, int E, int k, uint32_t flags,
                      int32_t* topk_expert, float* topk_prob, int32_t* split_sizes,
                      int32_t* expert_offsets, int32_t* dest_row, int32_t* src_token,
                      hipStream_t stream) {
    if (!split_sizes || !expert_offsets) return MOE_ERR_NULL;
    if (T > 0 && (!logits || !topk_expert || !topk_prob || !dest_row || !src_token))
        return MOE_ERR_NULL;
    if (T < 0 || E < 1 || E > kMaxExperts || k < 1 || k > E || T * k > INT32_MAX)
        return MOE_ERR_SHAPE;
    if (flags > MOE_ROUTE_SOFTMAX_ALL) return MOE_ERR_ARG;
    if (route_workspace_bytes(T, E, k) > kRouteScratchBytes) return MOE_ERR_WORKSPACE;
    if (!device_ok()) return MOE_ERR_UNSUPPORTED;
    void* ws = nullptr;
    if (route_scratch(&ws) != hipSuccess) return MOE_ERR_HIP;
    return hip_status(launch_route(logits, (int)T, E, k, flags, topk_expert, topk_prob,
                                   split_sizes, expert_offsets, dest_row, src_token, ws, stream));
}

int moe_router_fwd(const uint16_t* x, const uint16_t* w_router, int64_t T, int H, int E, int k,
                   uint32_t flags, float* logits, int32_t* topk_expert, float* topk_prob,
                   int32_t* split_sizes, int32_t* expert_offsets, int32_t* dest_row,
                   int32_t* src_token, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
    if (T < 0 || E < 1 || E > kMaxExperts || k < 1 || k > E || T * k > INT32_MAX || H < 64 ||
        (H % 64))
        return MOE_ERR_SHAPE;
    if (flags > MOE_ROUTE_SOFTMAX_ALL) return MOE_ERR_ARG;
    if (!split_sizes || !expert_offsets || !workspace) return MOE_ERR_NULL;
    if (T > 0 && (!x || !w_router || !logits || !topk_expert || !topk_prob || !dest_row ||
                  !src_token))
        return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(w_router)) return MOE_ERR_ALIGN;
    if (workspace_bytes < route_workspace_bytes(T, E, k)) return MOE_ERR_WORKSPACE;
    if (!device_ok()) return MOE_ERR_UNSUPPORTED;
    hipError_t e = launch_router_logits(x, w_router, (int)T, H, E, logits, stream);
    if (e != hipSuccess) return MOE_ERR_HIP;
    return hip_status(launch_route(logits, (int)T, E, k, flags, topk_expert, topk_prob,
                                   split_sizes, expert_offsets, dest_row, src_token, workspace,
                                   stream));
}

int moe_router_bwd(const float* dlogits, const uint16_t* x, const uint16_t* w_router, int64_t T,
                   int H, int E, int k, const int32_t* dest_row, const uint16_t* dxp,
                   uint16_t* dx, uint16_t* dw_router, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
    if (T < 0 || E < 1 || E > kMaxExperts || k < 1 || k > E || T * k > INT32_MAX || H < 64 ||
        (H % 64))
        return MOE_ERR_SHAPE;
    if (!w_router || !dw_router || !workspace) return MOE_ERR_NULL;
    if (T > 0 && (!dlogits || !x || !dx || (dxp && !dest_row))) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(w_router) || !aligned16(dxp) || !aligned16(dx) ||
        !aligned16(dw_router))
        return MOE_ERR_ALIGN;
    if (workspace_bytes < router_bwd_workspace_bytes(T, H, E)) return MOE_ERR_WORKSPACE;
    if (!device_ok()) return MOE_ERR_UNSUPPORTED;
    return hip_status(launch_router_bwd(dlogits, x, w_router, (int)T, H, E, k, dest_row, dxp, dx,
                                        dw_router, workspace, stream));
}

int moe_route_bwd(const float* topk_prob, const float* dprob_perm, const int32_t* dest_row,
                  const int32_t* topk_expert, const float* logits, int64_t T, int E, int k,
                  uint32_t flags, float* dlogits, hipStream_t stream) {
    if (T < 0 || E < 1 || E > kMaxExperts || k < 1 || k > E || T * k > INT32_MAX)
        return MOE_ERR_SHAPE;
    if (flags > MOE_ROUTE_SOFTMAX_ALL) return MOE_ERR_ARG;
    if (T > 0 && (!topk_prob || !dprob_perm || !dest_row || !topk_expert || !dlogits))
        return MOE_ERR_NULL;
    if (T > 0 && (flags & MOE_ROUTE_SOFTMAX_ALL) && !logits) return MOE_ERR_NULL;
    if (!device_ok()) return MOE_ERR_UNSUPPORTED;
    return hip_status(launch_route_bwd(topk_prob, dprob_perm, dest_row, topk_expert, logits,
                                       (int)T, E, k, flags, dlogits, stream));
}

int moe_check_routing(const int32_t* split_sizes, int E, int64_t rows, const int32_t* dest_row,
                      const int32_t* src_token, const int32_t* topk_expert, int64_t T, int k,
                      int32_t* status, hipStream_t stream) {
    if (!status) return MOE_ERR_NULL;
    if (T < 0 || rows < 0 || E < 1 || E > kMaxExperts) return MOE_ERR_SHAPE;
    if ((dest_row || topk_expert) && (k < 1 || k > E || T * k > INT32_MAX)) return MOE_ERR_SHAPE;
    if (!device_ok()) return MOE_ERR_UNSUPPORTED;
    return hip_status(launch_check_routing(split_sizes, E, rows, dest_row, src_token, topk_expert,
                                           T, k, status, stream));
}

int moe_permute(const uint16_t* x, int64_t T, int H, int k, const int32_t* dest_row,
                const float* topk_prob, uint16_t* xp, float* prob_perm, hipStream_t stream) {
    if (T < 0 || H < 8 || (H % 8) || k < 1 || k > kMaxTopK || T * k > INT32_MAX)
        return MOE_ERR_SHAPE;
    // x and xp both NULL: only the probabilities move (the rows are gathered
    // by the consumer, grouped_mlp_*_gather)
    if (T > 0 && (x == nullptr) != (xp == nullptr)) return MOE_ERR_NULL;
    if (T > 0 && !dest_row) return MOE_ERR_NULL;
    if (T > 0 && !x && (!topk_prob || !prob_perm)) return MOE_ERR_NULL;
    if (T > 0 && topk_prob && !prob_perm) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(xp)) return MOE_ERR_ALIGN;
    if (!device_ok()) return MOE_ERR_UNSUPPORTED;
    return hip_status(launch_permute(x, (int)T, H, k, dest_row, topk_prob, xp, prob_perm, stream));
}

int moe_unpermute(const uint16_t* yp, int64_t T, int H, int k, const int32_t* dest_row,
                  const float* topk_prob, uint16_t* y, hipStream_t stream) {
    if (T < 0 || H < 8 || (H % 8) || k < 1 || k > kMaxTopK || T * k > INT32_MAX)
        return MOE_ERR_SHAPE;
    if (T > 0 && (!yp || !dest_row || !y)) return MOE_ERR_NULL;
    if (!aligned16(yp) || !aligned16(y)) return MOE_ERR_ALIGN;
    if (!device_ok()) return MOE_ERR_UNSUPPORTED;
    return hip_status(launch_unpermute(yp, (int)T, H, k, dest_row, topk_prob, y, stream));
}

void mxfp8_colwise_bytes(int64_t rows, int64_t cols, int ngroups, size_t* code_bytes,
                         size_t* scale_bytes) {
    int g = ngroups > 1 ? ngroups : 1;
    size_t prows = (size_t)(rows < 0 ? 0 : rows) + (size_t)31 * g;
    prows = (prows + 31) / 32 * 32;
    if (code_bytes) *code_bytes = (size_t)(cols < 0 ? 0 : cols) * prows;
    if (scale_bytes) *scale_bytes = (size_t)(cols < 0 ? 0 : cols) * prows / 32;
}

static int check_quant_args(const void* a, const void* b, const void* c, int64_t rows,
                            int64_t cols, int axis, const int32_t* group_sizes, int ngroups) {
    if (axis != 0 && axis != 1) return MOE_ERR_ARG;
    if (rows < 0 || cols < 0 || rows > INT32_MAX) return MOE_ERR_SHAPE;
    if (axis == 1 && (cols % 32)) return MOE_ERR_SHAPE;
    if (axis == 0 && (cols % 8)) return MOE_ERR_SHAPE;
    if (axis == 0 && group_sizes && (ngroups < 1 || ngroups > kMaxExperts)) return MOE_ERR_SHAPE;
    if (rows > 0 && cols > 0 && (!a || !b || !c)) return MOE_ERR_NULL;
    if (!aligned16(a) || !aligned16(b)) return MOE_ERR_ALIGN;
    return MOE_OK;
}

int mxfp8_quantize(const uint16_t* x, int64_t rows, int64_t cols, int axis,
                   const int32_t* group_sizes, int ngroups, uint8_t* codes, uint8_t* scales,
                   hipStream_t stream) {
    int st = check_quant_args(x, codes, scales, rows, cols, axis, group_sizes, ngroups);
    if (st != MOE_OK) return st;
    if (!device_ok()) return MOE_ERR_UNSUPPORTED;
    MatTable src{}, c{}, s{};
    src.p[0] = x;
    c.p[0] = codes;
    s.p[0] = scales;
    if (axis == 1) return hip_status(launch_quant_rows(src, c, s, 1, rows, cols, stream));
    return hip_status(launch_quant_cols(src, c, s, 1, group_sizes, group_sizes ? ngroups : 1,
                                        rows, cols, stream));
}

int mxfp8_quantize_both(const uint16_t* x, int64_t rows, int64_t cols,
                        const int32_t* group_sizes, int ngroups, uint8_t* row_codes,
                        uint8_t* row_scales, uint8_t* col_codes, uint8_t* col_scales,
                        hipStream_t stream) {
    int st = check_quant_args(x, row_codes, row_scales, rows, cols, 1, nullptr, 0);
    if (st != MOE_OK) return st;
    if ((st = check_quant_args(x, col_codes, col_scales, rows, cols, 0, group_sizes, ngroups)) !=
        MOE_OK)
        return st;
    if (!device_ok()) return MOE_ERR_UNSUPPORTED;
    MatTable src{}, rc{}, rs{}, cc{}, cs{};
    src.p[0] = x;
    rc.p[0] = row_codes;
    rs.p[0] = row_scales;
    cc.p[0] = col_codes;
    cs.p[0] = col_scales;
    return hip_status(launch_quant(src, 1, group_sizes, group_sizes ? ngroups : 1, rows, cols, &rc,
                                   &rs, false, &cc, &cs, false, stream, "mx_quant_both"));
}

int mxfp8_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                     int axis, const int32_t* group_sizes, int ngroups, uint16_t* out,
                     hipStream_t stream) {
    int st = check_quant_args(codes, out, scales, rows, cols, axis, group_sizes, ngroups);
    if (st != MOE_OK) return st;
    if (!device_ok()) return MOE_ERR_UNSUPPORTED;
    if (axis == 1)
        return hip_status(launch_dequant_rows(codes, scales, rows, cols, out, stream));
    return hip_status(launch_dequant_cols(codes, scales, group_sizes, group_sizes ? ngroups : 1,
                                          rows, cols, out, stream));
}

}  // extern "C"
