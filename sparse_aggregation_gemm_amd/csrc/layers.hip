// GCN and GraphSAGE-mean layers, forward and backward, composed from the
// SpMM and the MFMA products.
//
// GCN (CAGNET page, forward-propagation equation; Sylvie, "Forward
// Propagation"): Y = A H_ext W + b.  GraphSAGE-mean (Sylvie, first section:
// aggregate the neighbours, update with the node's own row):
// Y = [H_local | A_mean H_ext] W + b.  Out = ReLU(Y) when asked.
// Backward (CAGNET page: the same SpMM and dense primitives; Sylvie,
// "Backward Propagation": halo rows of the input gradient go back to their
// owners): G_Y = G_out * 1[Y > 0], dW, db and dH_ext = A^T (G_Y W^T).
//
// The products associate either way, (A H) W = A (H W), and the SpMM is
// bandwidth-bound with its cost proportional to its width, so a layer
// aggregates first when d_in <= d_out and transforms first otherwise:
//   aggregate first  : Z = A H;  Y = Z W + b  (Z saved for dW = Z^T G_Y)
//   transform first  : T = H W;  Y = A T + b  (bias/ReLU fused in the SpMM)
//                      backward: S = A^T G_Y;  dW = H^T S;  dH = S W^T
// For GraphSAGE the self term rides along: transform first computes
// [P | T] = H [W_self | W_neigh] in one product and adds P in the SpMM's
// epilogue; the backward takes dW_self = H_local^T G_Y, dW_neigh = H^T S and
// dH = [G_Y | S] [W_self ; W_neigh]^T.
#include <algorithm>

#include "ops.h"

namespace sag {
namespace {

inline bool aggregate_first(int64_t d_in, int64_t d_out) { return d_in <= d_out; }

struct LayerWs {
    void* fz = nullptr;    // fused aggregate -> transform
    size_t fz_bytes = 0;
    void* Bp = nullptr;
    void* t1 = nullptr;    // dense temporary
    void* t2 = nullptr;    // dense temporary
    void* spmm = nullptr;
    size_t spmm_bytes = 0;
    void* tn = nullptr;
    size_t tn_bytes = 0;
    size_t total = 0;
};

// Workspace layout shared by the size queries and the calls.
LayerWs carve(void* ws, size_t bytes, size_t bp, size_t t1, size_t t2, size_t sp, size_t tn, size_t fz = 0) {
    Carver c(ws, bytes);
    LayerWs w;
    w.fz = c.take<char>(fz);
    w.fz_bytes = fz;
    w.Bp = c.take<char>(bp);
    w.t1 = c.take<char>(t1);
    w.t2 = c.take<char>(t2);
    w.spmm = c.take<char>(sp);
    w.spmm_bytes = sp;
    w.tn = c.take<char>(tn);
    w.tn_bytes = tn;
    w.total = c.used();
    return w;
}

sag_status check_layer_common(const char* who, const sag_csr* A, const void* H, int64_t ldh, int64_t d_in,
                              const void* W, int64_t d_out, sag_dtype dt) {
    const std::string w(who);
    if (dt != SAG_F32 && dt != SAG_BF16) return fail(SAG_E_INVALID, w + ": bad dtype");
    if (d_in <= 0 || d_out <= 0) return fail(SAG_E_INVALID, w + ": widths must be positive");
    // the SpMM runs at min(d_in, d_out) and supports 256 vectors of 16 bytes
    if (std::min(d_in, d_out) > (dt == SAG_BF16 ? 2048 : 1024))
        return fail(SAG_E_UNSUPPORTED, w + ": width too large");
    SAG_TRY(check_csr(who, A));
    SAG_TRY(check_dense("layer H_ext", H, A->n_cols, d_in, ldh, dt));
    if (!W) return fail(SAG_E_INVALID, w + ": null W");
    return SAG_OK;
}

// ---- GCN ----------------------------------------------------------------------------

LayerWs gcn_fwd_ws(const sag_csr& A, int64_t d_in, int64_t d_out, sag_dtype dt, void* ws, size_t bytes) {
    const size_t bp = packed_b_bytes(d_in, 0, d_out, dt);
    if (aggregate_first(d_in, d_out)) {
        const size_t fz = agg_transform_fits(d_in, d_out, false, dt) ? agg_transform_ws_bytes(A, d_in, d_out, false, dt)
                                                                     : 0;
        return carve(ws, bytes, bp, 0, 0, spmm_ws_bytes(A, d_in), 0, fz);
    }
    return carve(ws, bytes, bp, dense_bytes(A.n_cols, d_out, dt), 0, spmm_ws_bytes(A, d_out), 0);
}

LayerWs gcn_bwd_ws(const sag_csr* AT, int64_t n_local, int64_t d_in, int64_t d_out, sag_dtype dt, void* ws,
                   size_t bytes) {
    const int64_t n_ext = AT ? AT->n_rows : n_local;
    const size_t bp = packed_b_bytes(d_out, 0, d_in, dt);
    if (aggregate_first(d_in, d_out)) {
        // t1 = dZ [n_local, d_in]; the TN reduction runs over n_local rows
        return carve(ws, bytes, bp, dense_bytes(n_local, d_in, dt), 0, AT ? spmm_ws_bytes(*AT, d_in) : 0,
                     gemm_tn_ws_bytes(n_local, ldv(d_in, dt), d_out, dt));
    }
    // t1 = G_Y [n_local, d_out]; t2 = S [n_ext, d_out]; the TN buffer also
    // serves the column sums of G_Y (a product with no A columns)
    const size_t tn1 = gemm_tn_ws_bytes(n_ext, ldv(d_in, dt), d_out, dt);
    const size_t tn2 = gemm_tn_ws_bytes(n_local, 0, d_out, dt);
    return carve(ws, bytes, bp, dense_bytes(n_local, d_out, dt), dense_bytes(n_ext, d_out, dt),
                 AT ? spmm_ws_bytes(*AT, d_out) : 0, tn1 > tn2 ? tn1 : tn2);
}

// ---- SAGE ---------------------------------------------------------------------------

LayerWs sage_fwd_ws(const sag_csr& A, int64_t d_in, int64_t d_out, sag_dtype dt, void* ws, size_t bytes) {
    if (aggregate_first(d_in, d_out)) {
        const size_t fz = agg_transform_fits(d_in, d_out, true, dt) ? agg_transform_ws_bytes(A, d_in, d_out, true, dt)
                                                                    : 0;
        return carve(ws, bytes, packed_b_bytes(d_in, d_in, d_out, dt), 0, 0, spmm_ws_bytes(A, d_in), 0, fz);
    }
    const int64_t np = ldv(d_out, dt);
    // t1 = [P | T], [n_ext, np + d_out]
    return carve(ws, bytes, packed_b_bytes(d_in, 0, np + d_out, dt), dense_bytes(A.n_cols, np + d_out, dt), 0,
                 spmm_ws_bytes(A, d_out), 0);
}

LayerWs sage_bwd_ws(const sag_csr* AT, int64_t n_local, int64_t d_in, int64_t d_out, sag_dtype dt, void* ws,
                    size_t bytes) {
    const int64_t n_ext = AT ? AT->n_rows : n_local;
    if (aggregate_first(d_in, d_out)) {
        const int64_t ip = ldv(d_in, dt);
        // t1 = [dH_self | dM], [n_local, ip + d_in]
        return carve(ws, bytes, packed_b_bytes(d_out, 0, ip + d_in, dt), dense_bytes(n_local, ip + d_in, dt), 0,
                     AT ? spmm_ws_bytes(*AT, d_in) : 0, gemm_tn_ws_bytes(n_local, 2 * ip, d_out, dt));
    }
    // t1 = G_Y [n_local, d_out]; t2 = S [n_ext, d_out]
    const size_t tn1 = gemm_tn_ws_bytes(n_local, ldv(d_in, dt), d_out, dt);
    const size_t tn2 = gemm_tn_ws_bytes(n_ext, ldv(d_in, dt), d_out, dt);
    return carve(ws, bytes, packed_b_bytes(d_out, d_out, d_in, dt), dense_bytes(n_local, d_out, dt),
                 dense_bytes(n_ext, d_out, dt), AT ? spmm_ws_bytes(*AT, d_out) : 0, tn1 > tn2 ? tn1 : tn2);
}

}  // namespace
}  // namespace sag

using namespace sag;

// ===================================== GCN =============================================

extern "C" size_t sag_gcn_save_bytes(int64_t n_local, int64_t d_in, int64_t d_out, sag_dtype dt) {
    if (n_local < 0 || d_in <= 0 || d_out <= 0) return 0;
    return aggregate_first(d_in, d_out) ? dense_bytes(n_local, d_in, dt) : 0;
}

extern "C" size_t sag_gcn_forward_workspace_bytes(const sag_csr* A, int64_t d_in, int64_t d_out, sag_dtype dt) {
    if (!A || d_in <= 0 || d_out <= 0) return 0;
    return gcn_fwd_ws(*A, d_in, d_out, dt, nullptr, 0).total;
}

extern "C" sag_status sag_gcn_layer_forward(const sag_csr* A, const void* H_ext, int64_t ldh, int64_t d_in,
                                            const void* W, const float* b, int64_t d_out, int relu,
                                            unsigned options, sag_dtype dt, void* Y_pre, void* Out, int64_t ldo,
                                            void* save, size_t save_bytes, void* ws, size_t ws_bytes,
                                            void* stream) {
    SAG_TRY(check_layer_common("gcn_forward", A, H_ext, ldh, d_in, W, d_out, dt));
    if (options & ~static_cast<unsigned>(SAG_LAYER_FUSED)) return fail(SAG_E_INVALID, "gcn_forward: unknown option");
    if (!nn_k_fits(d_in, 0, dt)) return fail(SAG_E_UNSUPPORTED, "gcn_forward: d_in too large for the transform");
    const int64_t n_l = A->n_rows;
    SAG_TRY(check_dense("gcn_forward Out", Out, n_l, d_out, ldo, dt));
    if (Y_pre) SAG_TRY(check_dense("gcn_forward Y_pre", Y_pre, n_l, d_out, ldo, dt));
    if (save_bytes < sag_gcn_save_bytes(n_l, d_in, d_out, dt) || (save_bytes && !save && n_l))
        return fail(SAG_E_WORKSPACE, "gcn_forward: save buffer too small");
    if (save && !aligned16(save)) return fail(SAG_E_ALIGN, "gcn_forward: save not 16-B aligned");
    const LayerWs need = gcn_fwd_ws(*A, d_in, d_out, dt, nullptr, 0);
    if (ws_bytes < need.total || !ws) return fail(SAG_E_WORKSPACE, "gcn_forward: workspace too small");
    if (!aligned16(ws)) return fail(SAG_E_ALIGN, "gcn_forward: workspace not 16-B aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    LayerWs w = gcn_fwd_ws(*A, d_in, d_out, dt, ws, ws_bytes);

    PackSrc src;
    src.p[0][0] = W;
    src.sk[0][0] = d_out;
    src.sn[0][0] = 1;
    NLayout nl;
    nl.n0 = nl.nsplit = d_out;
    SAG_TRY(pack_b(src, d_in, 0, nl, dt, w.Bp, s));
    Epilogue e;
    e.bias = b;
    e.relu = relu;
    e.pre = Y_pre;
    e.row_mean = A->row_mean != 0;
    if (aggregate_first(d_in, d_out)) {
        const int64_t ldz = ldv(d_in, dt);
        if ((options & SAG_LAYER_FUSED) && w.fz_bytes)
            return agg_transform_run(*A, H_ext, ldh, d_in, W, b, d_out, false, relu, dt, Y_pre, Out, ldo, save, ldz,
                                     w.fz, w.fz_bytes, s);
        Epilogue ez;
        ez.row_mean = A->row_mean != 0;
        SAG_TRY(spmm_run(*A, H_ext, ldh, dt, d_in, save, ldz, dt, ez, w.spmm, w.spmm_bytes, s));
        e.row_mean = 0;
        GemmA a;
        a.a1 = save; a.lda1 = ldz; a.k1 = d_in; a.m1 = n_l;
        return gemm_run(n_l, d_out, a, w.Bp, dt, Out, ldo, e, s);
    }
    const int64_t ldt = ldv(d_out, dt);
    GemmA a;
    a.a1 = H_ext; a.lda1 = ldh; a.k1 = d_in; a.m1 = A->n_cols;
    SAG_TRY(gemm_run(A->n_cols, full_width(ldt), a, w.Bp, dt, w.t1, ldt, Epilogue{}, s));
    return spmm_run(*A, w.t1, ldt, dt, d_out, Out, ldo, dt, e, w.spmm, w.spmm_bytes, s);
}

extern "C" size_t sag_gcn_backward_workspace_bytes(const sag_csr* AT, int64_t n_local, int64_t d_in, int64_t d_out,
                                                   sag_dtype dt) {
    if (n_local < 0 || d_in <= 0 || d_out <= 0) return 0;
    return gcn_bwd_ws(AT, n_local, d_in, d_out, dt, nullptr, 0).total;
}

extern "C" sag_status sag_gcn_layer_backward(const sag_csr* AT, int64_t n_local, const void* H_ext, int64_t ldh,
                                             int64_t d_in, const void* W, int64_t d_out, int relu, const void* Y,
                                             const void* G_out, int64_t ldg, float* dW, float* db, void* dH_ext,
                                             int64_t ldd, sag_dtype dt, const void* save, size_t save_bytes,
                                             void* ws, size_t ws_bytes, void* stream) {
    const bool agg = aggregate_first(d_in, d_out);
    if (dt != SAG_F32 && dt != SAG_BF16) return fail(SAG_E_INVALID, "gcn_backward: bad dtype");
    if (n_local < 0 || d_in <= 0 || d_out <= 0) return fail(SAG_E_INVALID, "gcn_backward: bad sizes");
    if (AT) {
        SAG_TRY(check_csr("gcn_backward", AT));
        if (AT->n_cols != n_local) return fail(SAG_E_INVALID, "gcn_backward: AT columns differ from n_local");
    } else if (dH_ext || !agg) {
        return fail(SAG_E_INVALID, "gcn_backward: AT is needed for dH_ext or a transform-first layer");
    }
    const int64_t n_ext = AT ? AT->n_rows : n_local;
    if (!W || !dW) return fail(SAG_E_INVALID, "gcn_backward: null W or dW");
    if ((dH_ext || !agg) && !nn_k_fits(d_out, 0, dt))
        return fail(SAG_E_UNSUPPORTED, "gcn_backward: d_out too large for the input-gradient product");
    SAG_TRY(check_dense("gcn_backward G_out", G_out, n_local, d_out, ldg, dt));
    if (relu) SAG_TRY(check_dense("gcn_backward Y", Y, n_local, d_out, ldg, dt));
    if (dH_ext) SAG_TRY(check_dense("gcn_backward dH_ext", dH_ext, n_ext, d_in, ldd, dt));
    if (agg) {
        if (save_bytes < sag_gcn_save_bytes(n_local, d_in, d_out, dt) || (n_local && !save))
            return fail(SAG_E_INVALID, "gcn_backward: missing saved aggregate");
    } else {
        SAG_TRY(check_dense("gcn_backward H_ext", H_ext, n_ext, d_in, ldh, dt));
    }
    const LayerWs need = gcn_bwd_ws(AT, n_local, d_in, d_out, dt, nullptr, 0);
    if (ws_bytes < need.total || !ws) return fail(SAG_E_WORKSPACE, "gcn_backward: workspace too small");
    if (!aligned16(ws)) return fail(SAG_E_ALIGN, "gcn_backward: workspace not 16-B aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    LayerWs w = gcn_bwd_ws(AT, n_local, d_in, d_out, dt, ws, ws_bytes);
    const void* mask = relu ? Y : nullptr;

    // B = W^T: element (k, n) = W[n, k], k < d_out, n < d_in
    PackSrc src;
    src.p[0][0] = W;
    src.sk[0][0] = 1;
    src.sn[0][0] = d_out;
    NLayout nl;
    nl.n0 = nl.nsplit = d_in;

    if (agg) {
        const int64_t ldz = ldv(d_in, dt);
        GemmA z;
        z.a1 = save; z.lda1 = ldz; z.k1 = d_in; z.m1 = n_local;
        SAG_TRY(gemm_tn_run(n_local, d_out, z, G_out, ldg, mask, ldg, dW, d_out, db, dt, w.tn, w.tn_bytes, s));
        if (!dH_ext) return SAG_OK;
        SAG_TRY(pack_b(src, d_out, 0, nl, dt, w.Bp, s));
        GemmA g;
        g.a1 = G_out; g.lda1 = ldg; g.k1 = d_out; g.m1 = n_local; g.mask = mask; g.ldmask = ldg;
        SAG_TRY(gemm_run(n_local, full_width(ldz), g, w.Bp, dt, w.t1, ldz, Epilogue{}, s));
        return spmm_run(*AT, w.t1, ldz, dt, d_in, dH_ext, ldd, dt, Epilogue{}, w.spmm, w.spmm_bytes, s);
    }
    // transform first: G_Y, S = A^T G_Y, dW = H^T S, db = colsum G_Y, dH = S W^T
    const int64_t ldt = ldv(d_out, dt);
    const void* GY = G_out;
    int64_t ldgy = ldg;
    if (relu) {
        SAG_TRY(relu_mask_run(n_local, d_out, G_out, ldg, Y, ldg, w.t1, ldt, dt, s));
        GY = w.t1;
        ldgy = ldt;
    }
    SAG_TRY(spmm_run(*AT, GY, ldgy, dt, d_out, w.t2, ldt, dt, Epilogue{}, w.spmm, w.spmm_bytes, s));
    GemmA h;
    h.a1 = H_ext; h.lda1 = ldh; h.k1 = d_in; h.m1 = n_ext;
    SAG_TRY(gemm_tn_run(n_ext, d_out, h, w.t2, ldt, nullptr, 0, dW, d_out, nullptr, dt, w.tn, w.tn_bytes, s));
    if (db) {
        // column sums of G_Y: a TN product with no A columns
        GemmA none;
        none.m1 = n_local;
        SAG_TRY(gemm_tn_run(n_local, d_out, none, GY, ldgy, nullptr, 0, nullptr, d_out, db, dt, w.tn, w.tn_bytes, s));
    }
    if (!dH_ext) return SAG_OK;
    SAG_TRY(pack_b(src, d_out, 0, nl, dt, w.Bp, s));
    GemmA sg;
    sg.a1 = w.t2; sg.lda1 = ldt; sg.k1 = d_out; sg.m1 = n_ext;
    return gemm_run(n_ext, d_in, sg, w.Bp, dt, dH_ext, ldd, Epilogue{}, s);
}

// ===================================== SAGE ============================================

extern "C" size_t sag_sage_save_bytes(int64_t n_local, int64_t d_in, int64_t d_out, sag_dtype dt) {
    if (n_local < 0 || d_in <= 0 || d_out <= 0) return 0;
    return aggregate_first(d_in, d_out) ? dense_bytes(n_local, d_in, dt) : 0;
}

extern "C" size_t sag_sage_forward_workspace_bytes(const sag_csr* A, int64_t d_in, int64_t d_out, sag_dtype dt) {
    if (!A || d_in <= 0 || d_out <= 0) return 0;
    return sage_fwd_ws(*A, d_in, d_out, dt, nullptr, 0).total;
}

extern "C" sag_status sag_sage_layer_forward(const sag_csr* A, const void* H_ext, int64_t ldh, int64_t d_in,
                                             const void* W, const float* b, int64_t d_out, int relu,
                                             unsigned options, sag_dtype dt, void* Y_pre, void* Out, int64_t ldo,
                                             void* save, size_t save_bytes, void* ws, size_t ws_bytes,
                                             void* stream) {
    SAG_TRY(check_layer_common("sage_forward", A, H_ext, ldh, d_in, W, d_out, dt));
    if (options & ~static_cast<unsigned>(SAG_LAYER_FUSED)) return fail(SAG_E_INVALID, "sage_forward: unknown option");
    if (!nn_k_fits(d_in, aggregate_first(d_in, d_out) ? d_in : 0, dt))
        return fail(SAG_E_UNSUPPORTED, "sage_forward: d_in too large for the transform");
    const int64_t n_l = A->n_rows;
    if (A->n_cols < n_l) return fail(SAG_E_INVALID, "sage_forward: fewer columns than local rows");
    SAG_TRY(check_dense("sage_forward Out", Out, n_l, d_out, ldo, dt));
    if (Y_pre) SAG_TRY(check_dense("sage_forward Y_pre", Y_pre, n_l, d_out, ldo, dt));
    if (save_bytes < sag_sage_save_bytes(n_l, d_in, d_out, dt) || (save_bytes && !save && n_l))
        return fail(SAG_E_WORKSPACE, "sage_forward: save buffer too small");
    if (save && !aligned16(save)) return fail(SAG_E_ALIGN, "sage_forward: save not 16-B aligned");
    const LayerWs need = sage_fwd_ws(*A, d_in, d_out, dt, nullptr, 0);
    if (ws_bytes < need.total || !ws) return fail(SAG_E_WORKSPACE, "sage_forward: workspace too small");
    if (!aligned16(ws)) return fail(SAG_E_ALIGN, "sage_forward: workspace not 16-B aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    LayerWs w = sage_fwd_ws(*A, d_in, d_out, dt, ws, ws_bytes);
    const int64_t es = elt_size(dt);
    const char* Wc = static_cast<const char*>(W);
    Epilogue e;
    e.bias = b;
    e.relu = relu;
    e.pre = Y_pre;
    if (aggregate_first(d_in, d_out)) {
        // B = W with K blocks [W_self ; W_neigh]
        PackSrc src;
        src.p[0][0] = W;
        src.sk[0][0] = d_out;
        src.sn[0][0] = 1;
        src.p[1][0] = Wc + d_in * d_out * es;
        src.sk[1][0] = d_out;
        src.sn[1][0] = 1;
        NLayout nl;
        nl.n0 = nl.nsplit = d_out;
        SAG_TRY(pack_b(src, d_in, d_in, nl, dt, w.Bp, s));
        const int64_t ldm = ldv(d_in, dt);
        if ((options & SAG_LAYER_FUSED) && w.fz_bytes)
            return agg_transform_run(*A, H_ext, ldh, d_in, W, b, d_out, true, relu, dt, Y_pre, Out, ldo, save, ldm,
                                     w.fz, w.fz_bytes, s);
        // (a row-mean CSR gives every entry of row r the value 1/len(r): the
        // SpMM then scales each row's sum instead of reading values)
        Epilogue em;
        em.row_mean = A->row_mean != 0;
        SAG_TRY(spmm_run(*A, H_ext, ldh, dt, d_in, save, ldm, dt, em, w.spmm, w.spmm_bytes, s));
        GemmA a;
        a.a1 = H_ext; a.lda1 = ldh; a.k1 = d_in; a.m1 = n_l;
        a.a2 = save; a.lda2 = ldm; a.k2 = d_in;
        return gemm_run(n_l, d_out, a, w.Bp, dt, Out, ldo, e, s);
    }
    // transform first: [T | P] = H_ext [W_neigh | W_self]; Out = A T + P + b
    // (T first, so a gathered row of T starts on a cache line)
    const int64_t np = ldv(d_out, dt);
    const int64_t ldpt = ldv(np + d_out, dt);
    PackSrc src;
    src.p[0][0] = Wc + d_in * d_out * es;
    src.sk[0][0] = d_out;
    src.sn[0][0] = 1;
    src.p[0][1] = W;
    src.sk[0][1] = d_out;
    src.sn[0][1] = 1;
    NLayout nl;
    nl.n0 = d_out;
    nl.nsplit = np;
    nl.n1 = d_out;
    SAG_TRY(pack_b(src, d_in, 0, nl, dt, w.Bp, s));
    GemmA a;
    a.a1 = H_ext; a.lda1 = ldh; a.k1 = d_in; a.m1 = A->n_cols;
    SAG_TRY(gemm_run(A->n_cols, full_width(ldpt), a, w.Bp, dt, w.t1, ldpt, Epilogue{}, s));
    e.addend = static_cast<const char*>(w.t1) + np * es;
    e.ld_add = ldpt;
    e.n_add = n_l;
    e.row_mean = A->row_mean != 0;
    return spmm_run(*A, w.t1, ldpt, dt, d_out, Out, ldo, dt, e, w.spmm, w.spmm_bytes, s);
}

extern "C" size_t sag_sage_backward_workspace_bytes(const sag_csr* AT, int64_t n_local, int64_t d_in, int64_t d_out,
                                                    sag_dtype dt) {
    if (n_local < 0 || d_in <= 0 || d_out <= 0) return 0;
    return sage_bwd_ws(AT, n_local, d_in, d_out, dt, nullptr, 0).total;
}

extern "C" sag_status sag_sage_layer_backward(const sag_csr* AT, int64_t n_local, const void* H_ext, int64_t ldh,
                                              int64_t d_in, const void* W, int64_t d_out, int relu, const void* Y,
                                              const void* G_out, int64_t ldg, float* dW, float* db, void* dH_ext,
                                              int64_t ldd, sag_dtype dt, const void* save, size_t save_bytes,
                                              void* ws, size_t ws_bytes, void* stream) {
    const bool agg = aggregate_first(d_in, d_out);
    if (dt != SAG_F32 && dt != SAG_BF16) return fail(SAG_E_INVALID, "sage_backward: bad dtype");
    if (n_local < 0 || d_in <= 0 || d_out <= 0) return fail(SAG_E_INVALID, "sage_backward: bad sizes");
    if (AT) {
        SAG_TRY(check_csr("sage_backward", AT));
        if (AT->n_cols != n_local) return fail(SAG_E_INVALID, "sage_backward: AT columns differ from n_local");
    } else if (dH_ext || !agg) {
        return fail(SAG_E_INVALID, "sage_backward: AT is needed for dH_ext or a transform-first layer");
    }
    const int64_t n_ext = AT ? AT->n_rows : n_local;
    if (!W || !dW) return fail(SAG_E_INVALID, "sage_backward: null W or dW");
    if (!nn_k_fits(d_out, agg ? 0 : d_out, dt))
        return fail(SAG_E_UNSUPPORTED, "sage_backward: d_out too large for the input-gradient product");
    SAG_TRY(check_dense("sage_backward H_ext", H_ext, agg ? n_local : n_ext, d_in, ldh, dt));
    SAG_TRY(check_dense("sage_backward G_out", G_out, n_local, d_out, ldg, dt));
    if (relu) SAG_TRY(check_dense("sage_backward Y", Y, n_local, d_out, ldg, dt));
    if (dH_ext) SAG_TRY(check_dense("sage_backward dH_ext", dH_ext, n_ext, d_in, ldd, dt));
    if (agg && (save_bytes < sag_sage_save_bytes(n_local, d_in, d_out, dt) || (n_local && !save)))
        return fail(SAG_E_INVALID, "sage_backward: missing saved aggregate");
    const LayerWs need = sage_bwd_ws(AT, n_local, d_in, d_out, dt, nullptr, 0);
    if (ws_bytes < need.total || !ws) return fail(SAG_E_WORKSPACE, "sage_backward: workspace too small");
    if (!aligned16(ws)) return fail(SAG_E_ALIGN, "sage_backward: workspace not 16-B aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    LayerWs w = sage_bwd_ws(AT, n_local, d_in, d_out, dt, ws, ws_bytes);
    const void* mask = relu ? Y : nullptr;
    const int64_t es = elt_size(dt);
    const char* Wc = static_cast<const char*>(W);
    float* dW_neigh = dW + d_in * d_out;

    if (agg) {
        const int64_t ldm = ldv(d_in, dt);
        GemmA x;
        x.a1 = H_ext; x.lda1 = ldh; x.k1 = d_in; x.m1 = n_local;
        x.a2 = save; x.lda2 = ldm; x.k2 = d_in;
        SAG_TRY(gemm_tn_run(n_local, d_out, x, G_out, ldg, mask, ldg, dW, d_out, db, dt, w.tn, w.tn_bytes, s));
        if (!dH_ext) return SAG_OK;
        // [dH_self | dM] = G_Y [W_self ; W_neigh]^T: element (k, n) of N block
        // t is W[t * d_in + n, k]
        const int64_t ip = ldv(d_in, dt);
        const int64_t ldx = ldv(ip + d_in, dt);
        PackSrc src;
        src.p[0][0] = W;
        src.sk[0][0] = 1;
        src.sn[0][0] = d_out;
        src.p[0][1] = Wc + d_in * d_out * es;
        src.sk[0][1] = 1;
        src.sn[0][1] = d_out;
        NLayout nl;
        nl.n0 = d_in;
        nl.nsplit = ip;
        nl.n1 = d_in;
        SAG_TRY(pack_b(src, d_out, 0, nl, dt, w.Bp, s));
        GemmA g;
        g.a1 = G_out; g.lda1 = ldg; g.k1 = d_out; g.m1 = n_local; g.mask = mask; g.ldmask = ldg;
        SAG_TRY(gemm_run(n_local, full_width(ldx), g, w.Bp, dt, w.t1, ldx, Epilogue{}, s));
        Epilogue e;
        e.addend = w.t1;
        e.ld_add = ldx;
        e.n_add = n_local;
        const void* dM = static_cast<const char*>(w.t1) + ip * es;
        return spmm_run(*AT, dM, ldx, dt, d_in, dH_ext, ldd, dt, e, w.spmm, w.spmm_bytes, s);
    }
    // transform first
    const int64_t ldt = ldv(d_out, dt);
    const void* GY = G_out;
    int64_t ldgy = ldg;
    if (relu) {
        SAG_TRY(relu_mask_run(n_local, d_out, G_out, ldg, Y, ldg, w.t1, ldt, dt, s));
        GY = w.t1;
        ldgy = ldt;
    }
    SAG_TRY(spmm_run(*AT, GY, ldgy, dt, d_out, w.t2, ldt, dt, Epilogue{}, w.spmm, w.spmm_bytes, s));
    GemmA hl;
    hl.a1 = H_ext; hl.lda1 = ldh; hl.k1 = d_in; hl.m1 = n_local;
    SAG_TRY(gemm_tn_run(n_local, d_out, hl, GY, ldgy, nullptr, 0, dW, d_out, db, dt, w.tn, w.tn_bytes, s));
    GemmA he;
    he.a1 = H_ext; he.lda1 = ldh; he.k1 = d_in; he.m1 = n_ext;
    SAG_TRY(gemm_tn_run(n_ext, d_out, he, w.t2, ldt, nullptr, 0, dW_neigh, d_out, nullptr, dt, w.tn, w.tn_bytes, s));
    if (!dH_ext) return SAG_OK;
    // dH = [G_Y | S] [W_self^T ; W_neigh^T]: element (k, n) of K block s is
    // W[s * d_in + n, k]
    PackSrc src;
    src.p[0][0] = W;
    src.sk[0][0] = 1;
    src.sn[0][0] = d_out;
    src.p[1][0] = Wc + d_in * d_out * es;
    src.sk[1][0] = 1;
    src.sn[1][0] = d_out;
    NLayout nl;
    nl.n0 = nl.nsplit = d_in;
    SAG_TRY(pack_b(src, d_out, d_out, nl, dt, w.Bp, s));
    GemmA g;
    g.a1 = GY; g.lda1 = ldgy; g.k1 = d_out; g.m1 = n_local;
    g.a2 = w.t2; g.lda2 = ldt; g.k2 = d_out;
    return gemm_run(n_ext, d_in, g, w.Bp, dt, dH_ext, ldd, Epilogue{}, s);
}
