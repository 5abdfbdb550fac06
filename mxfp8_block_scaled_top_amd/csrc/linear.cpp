// grouped_linear_fwd / grouped_linear_bwd: one linear map per expert over the
// expert's rows, in one grouped GEMM launch per pass [BioNeMo MoE recipe page,
// section GroupedLinear: the tokens of all local experts with split_sizes, each
// expert with its own weight, instead of one GEMM launch per expert].
//
// The launches reuse the grouped-MLP GEMM kernels with their plain-store
// epilogue:
//   forward   y_e  = x_e W_e^T      K-major operands (ragged rows)
//   dgrad     dx_e = dy_e W_e       MXFP8: W blocked along N, stored [K, N];
//                                   BF16: W read in its natural [N, K] order
//   wgrad     dW_e = dy_e^T x_e     contraction over the expert's rows
//                                   (ragged K; MXFP8: grouped columnwise
//                                   operands, 32-row blocks from each
//                                   expert's first row)
// MXFP8 mode quantizes every operand along the contraction axis of the GEMM
// that reads it, from bf16, inside the call.
#include "moe_mi355x.h"

#include <hip/hip_runtime.h>

#include "kernels.hpp"
#include "mlp.hpp"

using namespace moe;

namespace {

size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

struct Carve {
    uint8_t* p;
    size_t off = 0;
    explicit Carve(void* base) : p((uint8_t*)base) {}
    uint8_t* take(size_t n) {
        uint8_t* r = p ? p + off : nullptr;
        off += al(n);
        return r;
    }
};

size_t colwise_codes(int64_t rows, int64_t cols, int E) {
    size_t c = 0;
    mxfp8_colwise_bytes(rows, cols, E, &c, nullptr);
    return c;
}

struct LinFwdWs {
    uint8_t *xq, *xq_s, *wq, *wq_s;
    size_t bytes;
};

LinFwdWs carve_lin_fwd(void* base, int64_t rows, int N, int K, int E, int precision) {
    Carve c(base);
    LinFwdWs w{};
    if (precision == MOE_MXFP8) {   // 8-bit operands in the row-pair layout
        const int64_t rp = padded_rows(rows, E);
        w.xq = c.take(p2_bytes(rp, K));
        w.xq_s = c.take((size_t)rp * K / 32);
        w.wq = c.take((size_t)E * p2_bytes(N, K));
        w.wq_s = c.take((size_t)E * N * K / 32);
    }
    c.take(256);
    w.bytes = c.off;
    return w;
}

struct LinBwdWs {
    uint8_t *dyq, *dyq_s;   // dy blocked along N (dgrad)
    uint8_t *dyc, *dyc_s;   // dy grouped columnwise (wgrad)
    uint8_t *wc, *wc_s;     // W blocked along N: [E][K, N]
    uint8_t *xc, *xc_s;     // x grouped columnwise (wgrad)
    size_t bytes;
};

LinBwdWs carve_lin_bwd(void* base, int64_t rows, int N, int K, int E, int precision) {
    Carve c(base);
    LinBwdWs w{};
    if (precision == MOE_MXFP8) {   // 8-bit operands in the row-pair layout
        const int64_t rp = padded_rows(rows, E);
        w.dyq = c.take(p2_bytes(rp, N));
        w.dyq_s = c.take((size_t)rp * N / 32);
        const size_t cn = colwise_codes(rows, N, E), ck = colwise_codes(rows, K, E);
        w.dyc = c.take(grouped_p2_bytes(rows, N, E));
        w.dyc_s = c.take(cn / 32);
        w.wc = c.take((size_t)E * p2_bytes(K, N));
        w.wc_s = c.take((size_t)E * N * K / 32);
        w.xc = c.take(grouped_p2_bytes(rows, K, E));
        w.xc_s = c.take(ck / 32);
    }
    c.take(256);
    w.bytes = c.off;
    return w;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_linear(int precision, int E, int N, int K, int64_t rows) {
    if (precision != MOE_BF16 && precision != MOE_MXFP8) return MOE_ERR_ARG;
    if (E < 1 || E > kMaxExperts) return MOE_ERR_SHAPE;
    if (N < 32 || K < 32 || (N % 32) || (K % 32)) return MOE_ERR_SHAPE;
    if (rows < 0 || rows > INT32_MAX) return MOE_ERR_SHAPE;
    // offsets that span a whole tensor stay below 2^31: inside one bf16
    // weight, and inside the block-major scales of the 8-bit row operands
    const int64_t kMaxSpan = (int64_t)1 << 31;
    const int64_t widest = N > K ? N : K;
    if ((int64_t)N * K * 2 >= kMaxSpan) return MOE_ERR_SHAPE;
    if (widest / 32 * padded_rows(rows, E) >= kMaxSpan) return MOE_ERR_SHAPE;
    return MOE_OK;
}

}  // namespace

namespace moe {
size_t linear_fwd_workspace_bytes(int64_t rows, int N, int K, int E, int precision) {
    return carve_lin_fwd(nullptr, rows, N, K, E, precision).bytes;
}
size_t linear_bwd_workspace_bytes(int64_t rows, int N, int K, int E, int precision) {
    return carve_lin_bwd(nullptr, rows, N, K, E, precision).bytes;
}
}  // namespace moe

#define MOE_TRY(x)                                 \
    do {                                           \
        if ((x) != hipSuccess) return MOE_ERR_HIP; \
    } while (0)

extern "C" {

int grouped_linear_fwd(int precision, int E, int N, int K, int64_t rows, const uint16_t* x,
                       const int32_t* split_sizes, const uint16_t* const* w, uint16_t* y,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int st = check_linear(precision, E, N, K, rows);
    if (st != MOE_OK) return st;
    if (!split_sizes || !w || !workspace) return MOE_ERR_NULL;
    for (int e = 0; e < E; ++e) {
        if (!w[e]) return MOE_ERR_NULL;
        if (!aligned16(w[e])) return MOE_ERR_ALIGN;
    }
    if (rows > 0 && (!x || !y)) return MOE_ERR_NULL;
    if (!aligned16(x) || !aligned16(y)) return MOE_ERR_ALIGN;
    if (workspace_bytes < linear_fwd_workspace_bytes(rows, N, K, E, precision))
        return MOE_ERR_WORKSPACE;
    if (!moe_device_supported()) return MOE_ERR_UNSUPPORTED;
    if (rows == 0) return MOE_OK;

    GemmArgs g{};
    g.split = split_sizes;
    g.E = E;
    g.rows = rows;
    g.rows_pad = padded_rows(rows, E);
    g.N = N;
    g.K = K;
    g.c = y;
    g.ldc = N;
    g.lda = K;
    g.ldb = K;
    if (precision == MOE_BF16) {
        g.a = x;
        for (int e = 0; e < E; ++e) g.b.p[e] = w[e];
        g.name = "linear_bf16_fwd";
        MOE_TRY(launch_gemm(DT_BF16, U_DOWN_FWD, g, stream));
        return MOE_OK;
    }
    LinFwdWs ws = carve_lin_fwd(workspace, rows, N, K, E, precision);
    MatTable src{}, cd{}, sc{};
    src.p[0] = x;
    cd.p[0] = ws.xq;
    sc.p[0] = ws.xq_s;
    // x along K at the experts' padded rows (the group walk places them)
    MOE_TRY(launch_quant(src, 1, split_sizes, E, rows, K, &cd, &sc, true, nullptr, nullptr, false,
                         stream, "linear_mx_quant_x", nullptr, g.rows_pad));
    MatTable wt{}, wq{}, wsc{};
    for (int e = 0; e < E; ++e) {
        wt.p[e] = w[e];
        wq.p[e] = ws.wq + (size_t)e * p2_bytes(N, K);
        wsc.p[e] = ws.wq_s + (size_t)e * N * K / 32;
    }
    MOE_TRY(launch_quant_rows(wt, wq, wsc, E, N, K, stream, "linear_mx_quant_w", true, N));
    g.a = ws.xq;
    g.a_scale = ws.xq_s;
    g.lda_s = K / 32;
    g.b = wq;
    g.b_scale = wsc;
    g.ldb_s = K / 32;
    g.name = "linear_mx_fwd";
    MOE_TRY(launch_gemm(DT_MX, U_DOWN_FWD, g, stream));
    return MOE_OK;
}

int grouped_linear_bwd(int precision, int E, int N, int K, int64_t rows, const uint16_t* dy,
                       const uint16_t* x, const int32_t* split_sizes, const uint16_t* const* w,
                       uint16_t* dx, uint16_t* const* dw, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
    int st = check_linear(precision, E, N, K, rows);
    if (st != MOE_OK) return st;
    if (!split_sizes || !workspace) return MOE_ERR_NULL;
    if (dx && !w) return MOE_ERR_NULL;
    for (int e = 0; e < E; ++e) {
        if (dx && !w[e]) return MOE_ERR_NULL;
        if (dw && !dw[e]) return MOE_ERR_NULL;
        if ((dx && !aligned16(w[e])) || (dw && !aligned16(dw[e]))) return MOE_ERR_ALIGN;
    }
    if (rows > 0 && (!dy || (dw && !x))) return MOE_ERR_NULL;
    if (!aligned16(dy) || !aligned16(x) || !aligned16(dx)) return MOE_ERR_ALIGN;
    if (workspace_bytes < linear_bwd_workspace_bytes(rows, N, K, E, precision))
        return MOE_ERR_WORKSPACE;
    if (!moe_device_supported()) return MOE_ERR_UNSUPPORTED;

    MatTable dwt{};
    if (dw)
        for (int e = 0; e < E; ++e) dwt.p[e] = dw[e];
    GemmArgs dg{};   // dx_e = dy_e W_e: [rows, K], contraction over N
    dg.split = split_sizes;
    dg.E = E;
    dg.rows = rows;
    dg.rows_pad = padded_rows(rows, E);
    dg.N = K;
    dg.K = N;
    dg.c = dx;
    dg.ldc = K;
    dg.lda = N;
    GemmArgs wg{};   // dW_e = dy_e^T x_e: [N, K], contraction over the expert's rows
    wg.split = split_sizes;
    wg.E = E;
    wg.rows = rows;
    wg.rows_pad = dg.rows_pad;
    wg.M = N;
    wg.N = K;
    wg.c_tab = dwt;
    wg.ldc = K;
    if (precision == MOE_BF16) {
        if (dx && rows > 0) {
            dg.a = dy;
            for (int e = 0; e < E; ++e) dg.b.p[e] = w[e];   // [N, K] read as [K = N, N = K]
            dg.ldb = K;
            dg.name = "linear_bf16_dgrad";
            MOE_TRY(launch_gemm(DT_BF16, U_GATEUP_DGRAD, dg, stream));
        }
        if (dw) {
            wg.a = dy;
            wg.lda = N;
            wg.b.p[0] = x;
            wg.ldb = K;
            wg.name = "linear_bf16_wgrad";
            MOE_TRY(launch_gemm(DT_BF16, U_GATEUP_WGRAD, wg, stream));
        }
        return MOE_OK;
    }
    LinBwdWs ws = carve_lin_bwd(workspace, rows, N, K, E, precision);
    if (rows > 0) {
        // dy: along N for the data gradient, grouped columnwise for the
        // weight gradient, from one read
        MatTable src{}, rc{}, rs{}, cc{}, cs{};
        src.p[0] = dy;
        rc.p[0] = ws.dyq;
        rs.p[0] = ws.dyq_s;
        cc.p[0] = ws.dyc;
        cs.p[0] = ws.dyc_s;
        MOE_TRY(launch_quant(src, 1, split_sizes, E, rows, N, dx ? &rc : nullptr,
                             dx ? &rs : nullptr, true, dw ? &cc : nullptr, dw ? &cs : nullptr,
                             true, stream, "linear_mx_quant_dy", nullptr, dg.rows_pad));
    }
    if (dx && rows > 0) {
        MatTable wt{}, wc{}, wcs{};
        for (int e = 0; e < E; ++e) {
            wt.p[e] = w[e];
            wc.p[e] = ws.wc + (size_t)e * p2_bytes(K, N);
            wcs.p[e] = ws.wc_s + (size_t)e * N * K / 32;
        }
        // W_e [N, K] in 32-row blocks along N, stored [K, N]
        MOE_TRY(launch_quant_cols(wt, wc, wcs, E, nullptr, 1, N, K, stream, "linear_mx_quant_w",
                                  true, N));
        dg.a = ws.dyq;
        dg.a_scale = ws.dyq_s;
        dg.lda_s = N / 32;
        dg.b = wc;
        dg.ldb = N;
        dg.b_scale = wcs;
        dg.ldb_s = N / 32;
        dg.name = "linear_mx_dgrad";
        MOE_TRY(launch_gemm(DT_MX, U_GATEUP_DGRAD, dg, stream));
    }
    if (dw) {
        if (rows > 0) {
            MatTable src{}, cc{}, cs{};
            src.p[0] = x;
            cc.p[0] = ws.xc;
            cs.p[0] = ws.xc_s;
            MOE_TRY(launch_quant_cols(src, cc, cs, 1, split_sizes, E, rows, K, stream,
                                      "linear_mx_quant_x", true, dg.rows_pad));
        }
        wg.a = ws.dyc;
        wg.a_scale = ws.dyc_s;
        wg.b.p[0] = ws.xc;
        wg.b_scale.p[0] = ws.xc_s;
        wg.name = "linear_mx_wgrad";
        MOE_TRY(launch_gemm(DT_MX, U_GATEUP_WGRAD, wg, stream));
    }
    return MOE_OK;
}

}  // extern "C"
