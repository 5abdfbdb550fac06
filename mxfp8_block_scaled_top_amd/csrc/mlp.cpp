// grouped_mlp_fwd / grouped_mlp_bwd: the launch sequences of the grouped
// expert MLP and their workspace layouts.
//
// Forward (per expert e, all experts per launch):
//   gate_up GEMM  A1 = Xp W1^T  + ScaledSwiGLU epilogue (A1 saved as bf16;
//                 A2 = p silu(g) u written as bf16, or as rowwise + grouped
//                 columnwise MXFP8)
//   down GEMM     Yp = A2 W2^T
// Backward:
//   down dgrad    dA2 = dYp W2  + SwiGLU-backward epilogue (dA1 as bf16 or
//                 MXFP8 row + column, per-tile probability-gradient partials)
//   dprob reduce  fixed-order sum of the partials
//   down wgrad    dW2 = dYp^T A2       (ragged K = rows of the expert)
//   gate_up dgrad dXp = dA1 W1
//   gate_up wgrad dW1 = dA1^T Xp       (ragged K)
// MXFP8 mode first quantizes the GEMM operands that arrive in bf16 (Xp, dYp,
// both weight sets) along the contraction axis of the GEMM that reads them.
#include "moe_mi355x.h"

#include <hip/hip_runtime.h>
#include <string.h>

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

struct FwdWs {
    uint8_t *xq, *xq_s, *w1q, *w1q_s, *w2q, *w2q_s, *a2q, *a2q_s;
    // FP8: bf16 A2 before its cast, the tensor maxima (xp, W1_e, W2_e, A2), the
    // amax reduction's partials, and the gate_up GEMM's per-workgroup maxima of A2
    uint8_t *a2bf, *amax_ws;
    float* amax;
    uint32_t* a2_part;
    int a2_nparts;
    size_t bytes;
};

// 8-bit operands are stored in the row-pair layout (common.hpp); activation
// rows at their expert-padded positions (padded_rows(rows, E) of them).
FwdWs carve_fwd(void* base, int64_t rows, int H, int I, int E, int precision) {
    Carve c(base);
    FwdWs w{};
    if (precision != MOE_BF16) {
        const int64_t rp = padded_rows(rows, E);
        w.xq = c.take(p2_bytes(rp, H));
        w.xq_s = c.take((size_t)rp * H / 32);
        w.w1q = c.take((size_t)E * p2_bytes(2 * (int64_t)I, H));
        w.w1q_s = c.take((size_t)E * 2 * I * H / 32);
        w.w2q = c.take((size_t)E * p2_bytes(H, I));
        w.w2q_s = c.take((size_t)E * H * I / 32);
        w.a2q = c.take(p2_bytes(rp, I));
        w.a2q_s = c.take((size_t)rp * I / 32);
    }
    if (precision == MOE_FP8) {
        w.a2bf = c.take((size_t)rows * I * 2);
        w.amax = (float*)c.take((size_t)(2 * E + 2) * sizeof(float));
        w.amax_ws = c.take(amax_workspace_bytes(E));
        w.a2_nparts = (int)gemm_slots(G_M, EPI_SWIGLU_FWD, rows, E, 0, 2 * I, I);
        w.a2_part = (uint32_t*)c.take((size_t)w.a2_nparts * sizeof(uint32_t));
    }
    c.take(256);
    w.bytes = c.off;
    return w;
}

struct BwdWs {
    uint8_t *da1;           // bf16 [rows, 2I] (BF16 mode; FP8: before its cast)
    float* amax;            // FP8: maxima of dYp, W2_e, W1_e, dA1
    uint8_t* amax_ws;
    uint32_t* da1_part;     // FP8: the down dgrad GEMM's per-workgroup maxima of dA1
    int da1_nparts;
    uint8_t *dyq, *dyq_s;   // rowwise dYp
    uint8_t *dyc, *dyc_s;   // grouped columnwise dYp
    uint8_t *w2c, *w2c_s;   // W2 quantized along H: [E][I, H]
    uint8_t *w1c, *w1c_s;   // W1 quantized along 2I: [E][H, 2I]
    uint8_t *da1q, *da1q_s; // rowwise dA1 [rows, 2I]
    uint8_t *da1c, *da1c_s; // grouped columnwise dA1
    float* part;            // dprob partials [rows, ntiles]
    size_t bytes;
};

BwdWs carve_bwd(void* base, int64_t rows, int H, int I, int E, int precision) {
    Carve c(base);
    BwdWs w{};
    int ntn = gemm_n_tiles(EPI_SWIGLU_BWD, I, I);
    w.part = (float*)c.take((size_t)rows * ntn * sizeof(float));
    if (precision == MOE_BF16) {
        w.da1 = c.take((size_t)rows * 2 * I * 2);
    } else {
        const int64_t rp = padded_rows(rows, E);
        w.dyq = c.take(p2_bytes(rp, H));
        w.dyq_s = c.take((size_t)rp * H / 32);
        w.dyc = c.take(grouped_p2_bytes(rows, H, E));
        w.dyc_s = c.take(colwise_codes(rows, H, E) / 32);
        w.w2c = c.take((size_t)E * p2_bytes(I, H));
        w.w2c_s = c.take((size_t)E * H * I / 32);
        w.w1c = c.take((size_t)E * p2_bytes(H, 2 * (int64_t)I));
        w.w1c_s = c.take((size_t)E * 2 * I * H / 32);
        w.da1q = c.take(p2_bytes(rp, 2 * (int64_t)I));
        w.da1q_s = c.take((size_t)rp * 2 * I / 32);
        w.da1c = c.take(grouped_p2_bytes(rows, 2 * (int64_t)I, E));
        w.da1c_s = c.take(colwise_codes(rows, 2 * (int64_t)I, E) / 32);
    }
    if (precision == MOE_FP8) {
        w.da1 = c.take((size_t)rows * 2 * I * 2);
        w.amax = (float*)c.take((size_t)(2 * E + 2) * sizeof(float));
        w.amax_ws = c.take(amax_workspace_bytes(E));
        w.da1_nparts = (int)gemm_slots(G_M, EPI_SWIGLU_BWD, rows, E, 0, I, I);
        w.da1_part = (uint32_t*)c.take((size_t)w.da1_nparts * sizeof(uint32_t));
    }
    c.take(256);
    w.bytes = c.off;
    return w;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The optional columnwise MXFP8 copies of the weights in moe_saved: all four
// buffers or none, 16-byte aligned.
int check_weight_cols(const moe_saved* s) {
    const void* p[4] = {s->w_gate_up_col_codes, s->w_gate_up_col_scales, s->w_down_col_codes,
                        s->w_down_col_scales};
    int n = 0;
    for (const void* q : p) {
        n += q != nullptr;
        if (!aligned16(q)) return MOE_ERR_ALIGN;
    }
    return (n == 0 || n == 4) ? MOE_OK : MOE_ERR_ARG;
}

struct WeightCols {
    MatTable w1c, w1s, w2c, w2s;
};

// Per-expert slices: W1_e along 2I as [H, 2I] with block-major scales
// [2I/32][H]; W2_e along H as [I, H] with scales [H/32][I].
WeightCols weight_cols(const moe_saved* s, int E, int H, int I) {
    WeightCols w{};
    for (int e = 0; e < E; ++e) {
        w.w1c.p[e] = s->w_gate_up_col_codes + (size_t)e * 2 * I * H;
        w.w1s.p[e] = s->w_gate_up_col_scales + (size_t)e * 2 * I * H / 32;
        w.w2c.p[e] = s->w_down_col_codes + (size_t)e * H * I;
        w.w2s.p[e] = s->w_down_col_scales + (size_t)e * H * I / 32;
    }
    return w;
}

int check_common(int precision, int E, int H, int I, int64_t rows) {
    if (precision != MOE_BF16 && precision != MOE_MXFP8 && precision != MOE_FP8)
        return MOE_ERR_ARG;
    if (E < 1 || E > kMaxExperts) return MOE_ERR_SHAPE;
    if (H < 128 || I < 128 || (H % 128) || (I % 128)) return MOE_ERR_SHAPE;
    if (rows < 0 || rows > INT32_MAX) return MOE_ERR_SHAPE;
    // The GEMM kernels take their operands' buffer bases per tile (activations)
    // or per K step (M/N-contiguous operands), so only two offsets still span a
    // whole tensor and must stay below 2^31: inside one expert's bf16 weight
    // [2I, H], and inside the block-major scales of the widest 8-bit
    // activation operand, [max(H, 2I)/32][padded rows].
    const int64_t kMaxSpan = (int64_t)1 << 31;
    const int64_t widest = H > 2 * (int64_t)I ? H : 2 * (int64_t)I;
    if (2 * (int64_t)I * H * 2 >= kMaxSpan) return MOE_ERR_SHAPE;
    if (widest / 32 * padded_rows(rows, E) >= kMaxSpan) return MOE_ERR_SHAPE;
    return MOE_OK;
}

int device_check() { return moe_device_supported() ? MOE_OK : MOE_ERR_UNSUPPORTED; }

}  // namespace

namespace moe {
int mlp_workspace_region(int op, int region, int64_t rows, int H, int I, int E, int precision,
                         size_t* offset, size_t* bytes) {
    if (!offset || !bytes) return MOE_ERR_NULL;
    if (precision != MOE_MXFP8 && precision != MOE_FP8) return MOE_ERR_ARG;
    if (rows < 0 || E < 1 || E > kMaxExperts || H < 1 || I < 1) return MOE_ERR_SHAPE;
    const int64_t rp = padded_rows(rows, E);
    const size_t w1 = (size_t)E * 2 * I * H, w2 = (size_t)E * H * I;
    const uint8_t* p = nullptr;
    size_t n = 0;
    if (op == MOE_OP_MLP_FWD) {
        // carved from a non-null base (256) so that every region gets a pointer
        FwdWs o = carve_fwd((void*)(uintptr_t)256, rows, H, I, E, precision);
        switch (region) {
            case MOE_WS_XP_CODES: p = o.xq; n = p2_bytes(rp, H); break;
            case MOE_WS_XP_SCALES: p = o.xq_s; n = (size_t)rp * H / 32; break;
            case MOE_WS_W1_CODES: p = o.w1q; n = (size_t)E * p2_bytes(2 * (int64_t)I, H); break;
            case MOE_WS_W1_SCALES: p = o.w1q_s; n = w1 / 32; break;
            case MOE_WS_W2_CODES: p = o.w2q; n = (size_t)E * p2_bytes(H, I); break;
            case MOE_WS_W2_SCALES: p = o.w2q_s; n = w2 / 32; break;
            case MOE_WS_A2_CODES: p = o.a2q; n = p2_bytes(rp, I); break;
            case MOE_WS_A2_SCALES: p = o.a2q_s; n = (size_t)rp * I / 32; break;
            default: return MOE_ERR_ARG;
        }
    } else if (op == MOE_OP_MLP_BWD) {
        BwdWs o = carve_bwd((void*)(uintptr_t)256, rows, H, I, E, precision);
        const size_t ch = colwise_codes(rows, H, E), ci = colwise_codes(rows, 2 * (int64_t)I, E);
        switch (region) {
            case MOE_WS_DYP_CODES: p = o.dyq; n = p2_bytes(rp, H); break;
            case MOE_WS_DYP_SCALES: p = o.dyq_s; n = (size_t)rp * H / 32; break;
            case MOE_WS_DYP_COL_CODES: p = o.dyc; n = grouped_p2_bytes(rows, H, E); break;
            case MOE_WS_DYP_COL_SCALES: p = o.dyc_s; n = ch / 32; break;
            case MOE_WS_W2_COL_CODES: p = o.w2c; n = (size_t)E * p2_bytes(I, H); break;
            case MOE_WS_W2_COL_SCALES: p = o.w2c_s; n = w2 / 32; break;
            case MOE_WS_W1_COL_CODES: p = o.w1c; n = (size_t)E * p2_bytes(H, 2 * (int64_t)I); break;
            case MOE_WS_W1_COL_SCALES: p = o.w1c_s; n = w1 / 32; break;
            case MOE_WS_DA1_CODES: p = o.da1q; n = p2_bytes(rp, 2 * (int64_t)I); break;
            case MOE_WS_DA1_SCALES: p = o.da1q_s; n = (size_t)rp * 2 * I / 32; break;
            case MOE_WS_DA1_COL_CODES: p = o.da1c; n = grouped_p2_bytes(rows, 2 * (int64_t)I, E); break;
            case MOE_WS_DA1_COL_SCALES: p = o.da1c_s; n = ci / 32; break;
            default: return MOE_ERR_ARG;
        }
    } else {
        return MOE_ERR_ARG;
    }
    if (!p) return MOE_ERR_ARG;
    *offset = (size_t)((uintptr_t)p - 256);
    *bytes = n;
    return MOE_OK;
}

size_t mlp_saved_bytes(int precision, int member, int64_t rows, int H, int I, int E) {
    if (rows < 0 || E < 1 || E > kMaxExperts || H < 1 || I < 1) return 0;
    const bool q8 = precision == MOE_MXFP8 || precision == MOE_FP8;
    if (!q8 && precision != MOE_BF16) return 0;
    switch (member) {
        case 0: return (size_t)rows * 2 * I * 2;                         // a1
        case 1: return q8 ? 0 : (size_t)rows * I * 2;                    // a2
        case 2: return q8 ? grouped_p2_bytes(rows, I, E) : 0;            // a2_col_codes
        case 3: return q8 ? colwise_codes(rows, I, E) / 32 : 0;          // a2_col_scales
        case 4: return q8 ? grouped_p2_bytes(rows, H, E) : 0;            // xp_col_codes
        case 5: return q8 ? colwise_codes(rows, H, E) / 32 : 0;          // xp_col_scales
        case 6: return q8 ? (size_t)E * p2_bytes(H, 2 * (int64_t)I) : 0; // w_gate_up_col_codes
        case 7: return q8 ? (size_t)E * 2 * I * H / 32 : 0;              // w_gate_up_col_scales
        case 8: return q8 ? (size_t)E * p2_bytes(I, H) : 0;              // w_down_col_codes
        case 9: return q8 ? (size_t)E * H * I / 32 : 0;                  // w_down_col_scales
        default: return 0;
    }
}

size_t mlp_fwd_workspace_bytes(int64_t rows, int H, int I, int E, int precision) {
    return carve_fwd(nullptr, rows, H, I, E, precision).bytes;
}
size_t mlp_bwd_workspace_bytes(int64_t rows, int H, int I, int E, int precision) {
    return carve_bwd(nullptr, rows, H, I, E, precision).bytes;
}
}  // namespace moe

#define MOE_TRY(x)                               \
    do {                                         \
        if ((x) != hipSuccess) return MOE_ERR_HIP; \
    } while (0)

extern "C" {

int moe_workspace_region(int op, int region, int64_t rows, int H, int I, int E, int precision,
                         size_t* offset, size_t* bytes) {
    return mlp_workspace_region(op, region, rows, H, I, E, precision, offset, bytes);
}

size_t moe_saved_bytes(int precision, int member, int64_t rows, int H, int I, int E) {
    return mlp_saved_bytes(precision, member, rows, H, I, E);
}

}  // extern "C"

namespace {

// The forward of grouped_mlp_fwd (gather == NULL: xp holds the grouped rows)
// and of grouped_mlp_fwd_gather (grouped row r is row gather[r] of xp; 8-bit
// modes only, where xp is read only by the quantizer).
int mlp_fwd(int precision, int E, int H, int I, int64_t rows, const uint16_t* xp,
            const int32_t* gather, const int32_t* split_sizes, const uint16_t* const* w_gate_up,
            const uint16_t* const* w_down, const float* prob_perm, uint16_t* yp,
            const moe_saved* saved, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int st = check_common(precision, E, H, I, rows);
    if (st != MOE_OK) return st;
    if (!split_sizes || !w_gate_up || !w_down || !saved || !workspace) return MOE_ERR_NULL;
    for (int e = 0; e < E; ++e)
        if (!w_gate_up[e] || !w_down[e]) return MOE_ERR_NULL;
    if (rows > 0) {
        if (!xp || !prob_perm || !yp || !saved->a1) return MOE_ERR_NULL;
        if (precision == MOE_BF16 && !saved->a2) return MOE_ERR_NULL;
        if (precision != MOE_BF16 && (!saved->a2_col_codes || !saved->a2_col_scales ||
                                      !saved->xp_col_codes || !saved->xp_col_scales))
            return MOE_ERR_NULL;
    }
    if ((st = check_weight_cols(saved)) != MOE_OK) return st;
    if (!aligned16(xp) || !aligned16(yp) || !aligned16(saved->a1) || !aligned16(saved->a2))
        return MOE_ERR_ALIGN;
    for (int e = 0; e < E; ++e)
        if (!aligned16(w_gate_up[e]) || !aligned16(w_down[e])) return MOE_ERR_ALIGN;
    if (workspace_bytes < mlp_fwd_workspace_bytes(rows, H, I, E, precision))
        return MOE_ERR_WORKSPACE;
    if ((st = device_check()) != MOE_OK) return st;
    if (rows == 0) return MOE_OK;

    FwdWs w = carve_fwd(workspace, rows, H, I, E, precision);
    GemmArgs g{};
    g.split = split_sizes;
    g.E = E;
    g.rows = rows;
    g.rows_pad = padded_rows(rows, E);
    g.prob = prob_perm;
    g.I = I;
    if (precision == MOE_BF16) {
        g.a = xp;
        g.lda = H;
        for (int e = 0; e < E; ++e) g.b.p[e] = w_gate_up[e];
        g.ldb = H;
        g.N = 2 * I;
        g.K = H;
        g.a1 = saved->a1;
        g.act = saved->a2;
        g.name = "gemm_bf16_gateup_fwd_swiglu";
        MOE_TRY(launch_gemm(DT_BF16, U_GATEUP_FWD, g, stream));
        GemmArgs d = g;
        d.a = saved->a2;
        d.lda = I;
        for (int e = 0; e < E; ++e) d.b.p[e] = w_down[e];
        d.ldb = I;
        d.N = H;
        d.K = I;
        d.c = yp;
        d.ldc = H;
        d.name = "gemm_bf16_down_fwd";
        MOE_TRY(launch_gemm(DT_BF16, U_DOWN_FWD, d, stream));
        return MOE_OK;
    }
    // MXFP8: quantize operands along their contraction axis.  xp: rowwise for
    // gate_up, grouped columnwise (saved) for the gate_up weight gradient, from
    // one read.  FP8: the same casts with one scale per tensor, from its amax.
    const bool fp8 = precision == MOE_FP8;
    const int dt8 = fp8 ? DT_FP8 : DT_MX;
    MatTable src{}, cd{}, sc{}, ccd{}, csc{};
    src.p[0] = xp;
    cd.p[0] = w.xq;
    sc.p[0] = w.xq_s;
    ccd.p[0] = saved->xp_col_codes;
    csc.p[0] = saved->xp_col_scales;
    if (fp8 && gather)
        MOE_TRY(launch_amax_gather(xp, gather, rows, H, w.amax_ws, w.amax, stream, "fp8_amax_xp"));
    else if (fp8)
        MOE_TRY(launch_amax(src, 1, rows * H, w.amax_ws, w.amax, stream, "fp8_amax_xp"));
    const int64_t rpad = padded_rows(rows, E);
    MOE_TRY(launch_quant(src, 1, split_sizes, E, rows, H, &cd, &sc, true, &ccd, &csc, true, stream,
                         fp8 ? "fp8_quant_xp" : "mx_quant_xp", fp8 ? w.amax : nullptr, rpad,
                         gather));
    // weights: rowwise (along H for W1, along I for W2) for these GEMMs; with
    // the saved columnwise buffers, also the backward's copies from the same read
    MatTable w1t{}, w1c{}, w1s{}, w2t{}, w2c{}, w2s{};
    for (int e = 0; e < E; ++e) {
        w1t.p[e] = w_gate_up[e];
        w1c.p[e] = w.w1q + (size_t)e * 2 * I * H;
        w1s.p[e] = w.w1q_s + (size_t)e * 2 * I * H / 32;
        w2t.p[e] = w_down[e];
        w2c.p[e] = w.w2q + (size_t)e * H * I;
        w2s.p[e] = w.w2q_s + (size_t)e * H * I / 32;
    }
    const float* aw1 = fp8 ? w.amax + 1 : nullptr;       // per-expert tensor maxima
    const float* aw2 = fp8 ? w.amax + 1 + E : nullptr;
    if (fp8) {
        MOE_TRY(launch_amax(w1t, E, 2 * (int64_t)I * H, w.amax_ws, w.amax + 1, stream,
                            "fp8_amax_w1"));
        MOE_TRY(launch_amax(w2t, E, (int64_t)H * I, w.amax_ws, w.amax + 1 + E, stream,
                            "fp8_amax_w2"));
    }
    if (saved->w_gate_up_col_codes) {
        WeightCols wc = weight_cols(saved, E, H, I);
        MOE_TRY(launch_quant(w1t, E, nullptr, 1, 2 * (int64_t)I, H, &w1c, &w1s, true, &wc.w1c,
                             &wc.w1s, true, stream, fp8 ? "fp8_quant_w1" : "mx_quant_w1", aw1,
                             2 * (int64_t)I));
        MOE_TRY(launch_quant(w2t, E, nullptr, 1, H, I, &w2c, &w2s, true, &wc.w2c, &wc.w2s, true,
                             stream, fp8 ? "fp8_quant_w2" : "mx_quant_w2", aw2, H));
    } else {
        MOE_TRY(launch_quant(w1t, E, nullptr, 1, 2 * (int64_t)I, H, &w1c, &w1s, true, nullptr,
                             nullptr, false, stream, fp8 ? "fp8_quant_rows_w1" : "mx_quant_rows_w1",
                             aw1, 2 * (int64_t)I));
        MOE_TRY(launch_quant(w2t, E, nullptr, 1, H, I, &w2c, &w2s, true, nullptr, nullptr, false,
                             stream, fp8 ? "fp8_quant_rows_w2" : "mx_quant_rows_w2", aw2, H));
    }

    g.a = w.xq;
    g.lda = H;
    g.a_scale = w.xq_s;
    g.lda_s = H / 32;
    g.b = w1c;
    g.ldb = H;
    g.b_scale = w1s;
    g.ldb_s = H / 32;
    g.N = 2 * I;
    g.K = H;
    g.a1 = saved->a1;
    if (fp8) {
        g.act = (bf16_t*)w.a2bf;
        g.amax_part = w.a2_part;
        g.name = "gemm_fp8_gateup_fwd_swiglu";
    } else {
        g.q_row = w.a2q;
        g.q_row_s = w.a2q_s;
        g.q_col = saved->a2_col_codes;
        g.q_col_s = saved->a2_col_scales;
        g.name = "gemm_mx_gateup_fwd_swiglu";
    }
    MOE_TRY(launch_gemm(dt8, U_GATEUP_FWD, g, stream));
    if (fp8) {   // A2: its amax, then rowwise (down GEMM) and grouped columnwise (saved)
        src.p[0] = w.a2bf;
        cd.p[0] = w.a2q;
        sc.p[0] = w.a2q_s;
        ccd.p[0] = saved->a2_col_codes;
        csc.p[0] = saved->a2_col_scales;
        float* aa2 = w.amax + 2 * E + 1;
        // the maximum from the GEMM epilogue's per-workgroup partials
        MOE_TRY(launch_amax_final(w.a2_part, w.a2_nparts, aa2, stream, "fp8_amax_a2"));
        MOE_TRY(launch_quant(src, 1, split_sizes, E, rows, I, &cd, &sc, true, &ccd, &csc, true,
                             stream, "fp8_quant_a2", aa2, rpad));
    }
    GemmArgs d{};
    d.split = split_sizes;
    d.E = E;
    d.rows = rows;
    d.rows_pad = padded_rows(rows, E);
    d.I = I;
    d.a = w.a2q;
    d.lda = I;
    d.a_scale = w.a2q_s;
    d.lda_s = I / 32;
    d.b = w2c;
    d.ldb = I;
    d.b_scale = w2s;
    d.ldb_s = I / 32;
    d.N = H;
    d.K = I;
    d.c = yp;
    d.ldc = H;
    d.name = fp8 ? "gemm_fp8_down_fwd" : "gemm_mx_down_fwd";
    MOE_TRY(launch_gemm(dt8, U_DOWN_FWD, d, stream));
    return MOE_OK;
}

// The backward of grouped_mlp_bwd (gather == NULL) and grouped_mlp_bwd_gather
// (grouped row r of dY is row gather[r] of dyp; 8-bit modes only).  xp is
// read by the BF16 weight gradient only.
int mlp_bwd(int precision, int E, int H, int I, int64_t rows, const uint16_t* dyp,
            const int32_t* gather, const uint16_t* xp, const int32_t* split_sizes,
            const uint16_t* const* w_gate_up, const uint16_t* const* w_down,
            const float* prob_perm, const moe_saved* saved, uint16_t* dxp,
            uint16_t* const* dw_gate_up, uint16_t* const* dw_down, float* dprob_perm,
            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    int st = check_common(precision, E, H, I, rows);
    if (st != MOE_OK) return st;
    if (!split_sizes || !w_gate_up || !w_down || !saved || !workspace || !dw_gate_up ||
        !dw_down)
        return MOE_ERR_NULL;
    for (int e = 0; e < E; ++e)
        if (!w_gate_up[e] || !w_down[e] || !dw_gate_up[e] || !dw_down[e]) return MOE_ERR_NULL;
    if (rows > 0) {
        if (!dyp || !prob_perm || !dxp || !dprob_perm || !saved->a1) return MOE_ERR_NULL;
        if (precision == MOE_BF16 && !xp) return MOE_ERR_NULL;
        if (precision == MOE_BF16 && !saved->a2) return MOE_ERR_NULL;
        if (precision != MOE_BF16 && (!saved->a2_col_codes || !saved->a2_col_scales ||
                                      !saved->xp_col_codes || !saved->xp_col_scales))
            return MOE_ERR_NULL;
    }
    if ((st = check_weight_cols(saved)) != MOE_OK) return st;
    if (!aligned16(dyp) || !aligned16(xp) || !aligned16(dxp) || !aligned16(saved->a1) ||
        !aligned16(saved->a2))
        return MOE_ERR_ALIGN;
    for (int e = 0; e < E; ++e)
        if (!aligned16(w_gate_up[e]) || !aligned16(w_down[e]) || !aligned16(dw_gate_up[e]) ||
            !aligned16(dw_down[e]))
            return MOE_ERR_ALIGN;
    if (workspace_bytes < mlp_bwd_workspace_bytes(rows, H, I, E, precision))
        return MOE_ERR_WORKSPACE;
    if ((st = device_check()) != MOE_OK) return st;

    BwdWs w = carve_bwd(workspace, rows, H, I, E, precision);
    const int ntn = gemm_n_tiles(EPI_SWIGLU_BWD, I, I);
    MatTable dw1{}, dw2{};
    for (int e = 0; e < E; ++e) {
        dw1.p[e] = dw_gate_up[e];
        dw2.p[e] = dw_down[e];
    }
    // weight-gradient GEMMs run for every expert (empty experts get zeros),
    // even when there are no rows at all
    if (precision == MOE_BF16) {
        GemmArgs g{};
        g.split = split_sizes;
        g.E = E;
        g.rows = rows;
        g.rows_pad = padded_rows(rows, E);
        g.prob = prob_perm;
        g.I = I;
        if (rows > 0) {
            // down dgrad + SwiGLU backward
            g.a = dyp;
            g.lda = H;
            for (int e = 0; e < E; ++e) g.b.p[e] = w_down[e];
            g.ldb = I;            // W2 [H, I] read as [K = H, N = I]
            g.N = I;
            g.K = H;
            g.a1 = saved->a1;
            g.act = (bf16_t*)w.da1;
            g.dprob_part = w.part;
            g.name = "gemm_bf16_down_dgrad_swiglu_bwd";
            MOE_TRY(launch_gemm(DT_BF16, U_DOWN_DGRAD, g, stream));
            MOE_TRY(launch_dprob_reduce(w.part, rows, ntn, dprob_perm, stream));
        }
        // down wgrad: dW2 [H, I] = dYp^T A2
        GemmArgs wg{};
        wg.split = split_sizes;
        wg.E = E;
        wg.rows = rows;
        wg.rows_pad = padded_rows(rows, E);
        wg.a = dyp;
        wg.lda = H;
        wg.b.p[0] = saved->a2;
        wg.ldb = I;
        wg.M = H;
        wg.N = I;
        wg.c_tab = dw2;
        wg.ldc = I;
        wg.name = "gemm_bf16_down_wgrad";
        MOE_TRY(launch_gemm(DT_BF16, U_DOWN_WGRAD, wg, stream));
        if (rows > 0) {
            // gate_up dgrad: dXp = dA1 W1
            GemmArgs dg{};
            dg.split = split_sizes;
            dg.E = E;
            dg.rows = rows;
            dg.rows_pad = padded_rows(rows, E);
            dg.a = w.da1;
            dg.lda = 2 * I;
            for (int e = 0; e < E; ++e) dg.b.p[e] = w_gate_up[e];
            dg.ldb = H;           // W1 [2I, H] read as [K = 2I, N = H]
            dg.N = H;
            dg.K = 2 * I;
            dg.c = dxp;
            dg.ldc = H;
            dg.name = "gemm_bf16_gateup_dgrad";
            MOE_TRY(launch_gemm(DT_BF16, U_GATEUP_DGRAD, dg, stream));
        }
        // gate_up wgrad: dW1 [2I, H] = dA1^T Xp
        GemmArgs wg1{};
        wg1.split = split_sizes;
        wg1.E = E;
        wg1.rows = rows;
        wg1.rows_pad = padded_rows(rows, E);
        wg1.a = w.da1;
        wg1.lda = 2 * I;
        wg1.b.p[0] = xp;
        wg1.ldb = H;
        wg1.M = 2 * I;
        wg1.N = H;
        wg1.c_tab = dw1;
        wg1.ldc = H;
        wg1.name = "gemm_bf16_gateup_wgrad";
        MOE_TRY(launch_gemm(DT_BF16, U_GATEUP_WGRAD, wg1, stream));
        return MOE_OK;
    }

    // ---- MXFP8 and FP8 (per-tensor scales from each tensor's amax)
    const bool fp8 = precision == MOE_FP8;
    const int dt8 = fp8 ? DT_FP8 : DT_MX;
    const int64_t rpad = padded_rows(rows, E);
    MatTable src{}, cd{}, sc{};
    if (rows > 0) {
        // rowwise for the down dgrad, grouped columnwise for the down wgrad
        MatTable ccd{}, csc{};
        src.p[0] = dyp;
        cd.p[0] = w.dyq;
        sc.p[0] = w.dyq_s;
        ccd.p[0] = w.dyc;
        csc.p[0] = w.dyc_s;
        if (fp8 && gather)
            MOE_TRY(launch_amax_gather(dyp, gather, rows, H, w.amax_ws, w.amax, stream,
                                       "fp8_amax_dyp"));
        else if (fp8)
            MOE_TRY(launch_amax(src, 1, rows * H, w.amax_ws, w.amax, stream, "fp8_amax_dyp"));
        MOE_TRY(launch_quant(src, 1, split_sizes, E, rows, H, &cd, &sc, true, &ccd, &csc, true,
                             stream, fp8 ? "fp8_quant_dyp" : "mx_quant_dyp",
                             fp8 ? w.amax : nullptr, rpad, gather));
    }
    MatTable w1t{}, w1c{}, w1s{}, w2t{}, w2c{}, w2s{};
    for (int e = 0; e < E; ++e) {
        w2t.p[e] = w_down[e];
        w2c.p[e] = w.w2c + (size_t)e * H * I;
        w2s.p[e] = w.w2c_s + (size_t)e * H * I / 32;
        w1t.p[e] = w_gate_up[e];
        w1c.p[e] = w.w1c + (size_t)e * 2 * I * H;
        w1s.p[e] = w.w1c_s + (size_t)e * 2 * I * H / 32;
    }
    if (saved->w_gate_up_col_codes) {   // made by the forward from the same weights
        WeightCols wc = weight_cols(saved, E, H, I);
        w1c = wc.w1c;
        w1s = wc.w1s;
        w2c = wc.w2c;
        w2s = wc.w2s;
    }
    if (rows > 0) {
        if (!saved->w_gate_up_col_codes) {
            // W2 [H, I] along H -> [I, H];  W1 [2I, H] along 2I -> [H, 2I]
            const float* aw2 = fp8 ? w.amax + 1 : nullptr;
            const float* aw1 = fp8 ? w.amax + 1 + E : nullptr;
            if (fp8) {
                MOE_TRY(launch_amax(w2t, E, (int64_t)H * I, w.amax_ws, w.amax + 1, stream,
                                    "fp8_amax_w2"));
                MOE_TRY(launch_amax(w1t, E, 2 * (int64_t)I * H, w.amax_ws, w.amax + 1 + E,
                                    stream, "fp8_amax_w1"));
            }
            MOE_TRY(launch_quant(w2t, E, nullptr, 1, H, I, nullptr, nullptr, false, &w2c, &w2s,
                                 true, stream, fp8 ? "fp8_quant_cols_w2" : "mx_quant_cols_w2",
                                 aw2, H));
            MOE_TRY(launch_quant(w1t, E, nullptr, 1, 2 * (int64_t)I, H, nullptr, nullptr, false,
                                 &w1c, &w1s, true, stream,
                                 fp8 ? "fp8_quant_cols_w1" : "mx_quant_cols_w1", aw1,
                                 2 * (int64_t)I));
        }
        GemmArgs g{};
        g.split = split_sizes;
        g.E = E;
        g.rows = rows;
        g.rows_pad = padded_rows(rows, E);
        g.prob = prob_perm;
        g.I = I;
        g.a = w.dyq;
        g.lda = H;
        g.a_scale = w.dyq_s;
        g.lda_s = H / 32;
        g.b = w2c;
        g.ldb = H;
        g.b_scale = w2s;
        g.ldb_s = H / 32;
        g.N = I;
        g.K = H;
        g.a1 = saved->a1;
        g.dprob_part = w.part;
        if (fp8) {
            g.act = (bf16_t*)w.da1;
            g.amax_part = w.da1_part;
            g.name = "gemm_fp8_down_dgrad_swiglu_bwd";
        } else {
            g.q_row = w.da1q;
            g.q_row_s = w.da1q_s;
            g.q_col = w.da1c;
            g.q_col_s = w.da1c_s;
            g.name = "gemm_mx_down_dgrad_swiglu_bwd";
        }
        MOE_TRY(launch_gemm(dt8, U_DOWN_DGRAD, g, stream));
        MOE_TRY(launch_dprob_reduce(w.part, rows, ntn, dprob_perm, stream));
        if (fp8) {   // dA1: its amax, then rowwise (gate_up dgrad) and grouped columnwise
            MatTable ccd{}, csc{};
            src.p[0] = w.da1;
            cd.p[0] = w.da1q;
            sc.p[0] = w.da1q_s;
            ccd.p[0] = w.da1c;
            csc.p[0] = w.da1c_s;
            float* ad = w.amax + 2 * E + 1;
            // the maximum from the GEMM epilogue's per-workgroup partials
            MOE_TRY(launch_amax_final(w.da1_part, w.da1_nparts, ad, stream, "fp8_amax_da1"));
            MOE_TRY(launch_quant(src, 1, split_sizes, E, rows, 2 * (int64_t)I, &cd, &sc, true,
                                 &ccd, &csc, true, stream, "fp8_quant_da1", ad, rpad));
        }
    }
    // down wgrad: dW2 [H, I] = dYp^T A2 over grouped columnwise operands
    GemmArgs wg{};
    wg.split = split_sizes;
    wg.E = E;
    wg.rows = rows;
    wg.rows_pad = padded_rows(rows, E);
    wg.a = w.dyc;
    wg.a_scale = w.dyc_s;
    wg.b.p[0] = saved->a2_col_codes;
    wg.b_scale.p[0] = saved->a2_col_scales;
    wg.M = H;
    wg.N = I;
    wg.c_tab = dw2;
    wg.ldc = I;
    wg.name = fp8 ? "gemm_fp8_down_wgrad" : "gemm_mx_down_wgrad";
    MOE_TRY(launch_gemm(dt8, U_DOWN_WGRAD, wg, stream));
    if (rows > 0) {
        GemmArgs dg{};
        dg.split = split_sizes;
        dg.E = E;
        dg.rows = rows;
        dg.rows_pad = padded_rows(rows, E);
        dg.a = w.da1q;
        dg.lda = 2 * I;
        dg.a_scale = w.da1q_s;
        dg.lda_s = 2 * I / 32;
        dg.b = w1c;
        dg.ldb = 2 * I;
        dg.b_scale = w1s;
        dg.ldb_s = 2 * I / 32;
        dg.N = H;
        dg.K = 2 * I;
        dg.c = dxp;
        dg.ldc = H;
        dg.name = fp8 ? "gemm_fp8_gateup_dgrad" : "gemm_mx_gateup_dgrad";
        MOE_TRY(launch_gemm(dt8, U_GATEUP_DGRAD, dg, stream));
    }
    GemmArgs wg1{};
    wg1.split = split_sizes;
    wg1.E = E;
    wg1.rows = rows;
    wg1.rows_pad = padded_rows(rows, E);
    wg1.a = w.da1c;
    wg1.a_scale = w.da1c_s;
    wg1.b.p[0] = saved->xp_col_codes;
    wg1.b_scale.p[0] = saved->xp_col_scales;
    wg1.M = 2 * I;
    wg1.N = H;
    wg1.c_tab = dw1;
    wg1.ldc = H;
    wg1.name = fp8 ? "gemm_fp8_gateup_wgrad" : "gemm_mx_gateup_wgrad";
    MOE_TRY(launch_gemm(dt8, U_GATEUP_WGRAD, wg1, stream));
    return MOE_OK;
}

}  // namespace

extern "C" {

int grouped_mlp_fwd(int precision, int E, int H, int I, int64_t rows, const uint16_t* xp,
                    const int32_t* split_sizes, const uint16_t* const* w_gate_up,
                    const uint16_t* const* w_down, const float* prob_perm, uint16_t* yp,
                    const moe_saved* saved, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
    return mlp_fwd(precision, E, H, I, rows, xp, nullptr, split_sizes, w_gate_up, w_down,
                   prob_perm, yp, saved, workspace, workspace_bytes, stream);
}

int grouped_mlp_fwd_gather(int precision, int E, int H, int I, int64_t rows, const uint16_t* x,
                           const int32_t* src_token, const int32_t* split_sizes,
                           const uint16_t* const* w_gate_up, const uint16_t* const* w_down,
                           const float* prob_perm, uint16_t* yp, const moe_saved* saved,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (precision == MOE_BF16) return MOE_ERR_ARG;
    if (rows > 0 && !src_token) return MOE_ERR_NULL;
    return mlp_fwd(precision, E, H, I, rows, x, src_token, split_sizes, w_gate_up, w_down,
                   prob_perm, yp, saved, workspace, workspace_bytes, stream);
}

int grouped_mlp_bwd(int precision, int E, int H, int I, int64_t rows, const uint16_t* dyp,
                    const uint16_t* xp, const int32_t* split_sizes,
                    const uint16_t* const* w_gate_up, const uint16_t* const* w_down,
                    const float* prob_perm, const moe_saved* saved, uint16_t* dxp,
                    uint16_t* const* dw_gate_up, uint16_t* const* dw_down, float* dprob_perm,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return mlp_bwd(precision, E, H, I, rows, dyp, nullptr, xp, split_sizes, w_gate_up, w_down,
                   prob_perm, saved, dxp, dw_gate_up, dw_down, dprob_perm, workspace,
                   workspace_bytes, stream);
}

int grouped_mlp_bwd_gather(int precision, int E, int H, int I, int64_t rows, const uint16_t* dy,
                           const int32_t* src_token, const int32_t* split_sizes,
                           const uint16_t* const* w_gate_up, const uint16_t* const* w_down,
                           const float* prob_perm, const moe_saved* saved, uint16_t* dxp,
                           uint16_t* const* dw_gate_up, uint16_t* const* dw_down,
                           float* dprob_perm, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
    if (precision == MOE_BF16) return MOE_ERR_ARG;
    if (rows > 0 && !src_token) return MOE_ERR_NULL;
    return mlp_bwd(precision, E, H, I, rows, dy, src_token, nullptr, split_sizes, w_gate_up,
                   w_down, prob_perm, saved, dxp, dw_gate_up, dw_down, dprob_perm, workspace,
                   workspace_bytes, stream);
}

}  // extern "C"
