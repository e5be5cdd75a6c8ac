// Graph intake: checks a topologically ordered node list over the primitive
// set and infers every node's shape and dtype.
//
// limn README, "The op set": the primitives and the dtype rules (equal
// dtypes for binary ops here: promotion between dtypes is a frontend concern,
// so a mixed pair is RV_E_DTYPE). "Reading the schedule": a reduce keeps its
// reduced dims with size 1. ASSIGN, and CUSTOM kernels other than the
// attention forward, are declined with a typed error (Tiki README, "Compile
// model code").
#include <algorithm>

#include "graph.hpp"

namespace rv {

bool is_elementwise(int op) {
    return op == RV_NEG || op == RV_EXP || op == RV_LOG || op == RV_SQRT || op == RV_RECIP || op == RV_CAST ||
           op == RV_ADD || op == RV_MUL || op == RV_CMPLT || op == RV_WHERE;
}

bool is_reduce(int op) { return op == RV_SUM || op == RV_MAX; }

static int arity(int op) {
    switch (op) {
        case RV_BUFFER: case RV_CONST: return 0;
        case RV_ADD: case RV_MUL: case RV_CMPLT: case RV_GATHER: return 2;
        case RV_WHERE: case RV_CUSTOM: case RV_SCATTER: return 3;
        default: return 1;
    }
}

bool pure_broadcast(const rv_view& v, const Shape& src, std::vector<int>* src_dim_of_view) {
    if (v.offset != 0) return false;
    for (int d = 0; d < v.ndim; ++d)
        if (v.mask_lo[d] != 0 || v.mask_hi[d] != v.shape[d]) return false;
    // contiguous strides of the source
    std::vector<int64_t> cs(src.size());
    int64_t s = 1;
    for (int d = (int)src.size() - 1; d >= 0; --d) {
        cs[d] = s;
        s *= src[d];
    }
    std::vector<int> map(v.ndim, -1);
    int next = 0;  // next source dim that may be matched (order preserved)
    std::vector<int> used(src.size(), 0);
    for (int dv = 0; dv < v.ndim; ++dv) {
        if (v.shape[dv] == 1 || v.strides[dv] == 0) continue;  // broadcast or size-1 dim
        int found = -1;
        for (int ds = next; ds < (int)src.size(); ++ds) {
            if (src[ds] == 1) continue;
            if (src[ds] == v.shape[dv] && cs[ds] == v.strides[dv]) found = ds;
            break;
        }
        if (found < 0) return false;
        map[dv] = found;
        used[found] = 1;
        next = found + 1;
    }
    for (size_t ds = 0; ds < src.size(); ++ds)
        if (src[ds] != 1 && !used[ds]) return false;
    if (src_dim_of_view) *src_dim_of_view = map;
    return true;
}

Graph intake(const rv_node* nodes, int32_t n, const int32_t* outputs, int32_t nout) {
    if (n <= 0 || !nodes) fail(RV_E_INVALID, "empty graph");
    if (nout <= 0 || !outputs) fail(RV_E_INVALID, "no outputs");
    Graph g;
    g.nodes.resize(n);
    for (int i = 0; i < n; ++i) {
        const rv_node& in = nodes[i];
        Node& nd = g.nodes[i];
        nd.op = in.op;
        if (in.op < 0 || in.op > RV_CUSTOM) fail(RV_E_INVALID, fmt("node %d: unknown op %d", i, in.op));
        if (in.op == RV_ASSIGN || (in.op == RV_CUSTOM && in.buf != RV_CUSTOM_SDPA_FWD))
            fail(RV_E_UNSUPPORTED_OP, fmt("node %d: %s%s is not supported by this library", i, op_name(in.op),
                                          in.op == RV_CUSTOM ? fmt(" kernel %d", in.buf).c_str() : ""));
        nd.nsrc = arity(in.op);
        for (int k = 0; k < nd.nsrc; ++k) {
            nd.src[k] = in.src[k];
            if (in.src[k] < 0 || in.src[k] >= i)
                fail(RV_E_INVALID, fmt("node %d (%s): source %d is not an earlier node", i, op_name(in.op), in.src[k]));
        }
        auto S = [&](int k) -> const Node& { return g.nodes[nd.src[k]]; };
        switch (in.op) {
            case RV_BUFFER:
                view_check(in.view);
                if (!view_is_contiguous(in.view))
                    fail(RV_E_INVALID, fmt("node %d: a BUFFER's view must be contiguous", i));
                if (!dtype_valid(in.dtype)) fail(RV_E_DTYPE, fmt("node %d: bad dtype %d", i, in.dtype));
                if (in.buf < 0) fail(RV_E_INVALID, fmt("node %d: negative buffer slot", i));
                nd.shape = view_shape(in.view);
                nd.dtype = in.dtype;
                nd.slot = in.buf;
                g.n_inputs = std::max(g.n_inputs, in.buf + 1);
                break;
            case RV_CONST:
                view_check(in.view);
                if (!dtype_valid(in.dtype)) fail(RV_E_DTYPE, fmt("node %d: bad dtype %d", i, in.dtype));
                nd.shape = view_shape(in.view);
                nd.dtype = in.dtype;
                nd.cval = in.cval;
                break;
            case RV_VIEW: {
                view_check(in.view);
                const Node& s = S(0);
                int64_t lo, hi;
                if (view_addr_range(in.view, &lo, &hi) && (lo < 0 || hi >= numel(s.shape)))
                    fail(RV_E_OUT_OF_BOUNDS,
                         fmt("node %d: the View can address elements [%lld, %lld] of a source with %lld elements", i,
                             (long long)lo, (long long)hi, (long long)numel(s.shape)));
                nd.shape = view_shape(in.view);
                nd.dtype = s.dtype;
                nd.view = in.view;
                break;
            }
            case RV_NEG: case RV_EXP: case RV_LOG: case RV_SQRT: case RV_RECIP:
                nd.shape = S(0).shape;
                nd.dtype = S(0).dtype;
                if (in.op != RV_NEG && !is_float(nd.dtype))
                    fail(RV_E_DTYPE, fmt("node %d: %s needs a float operand, got %s", i, op_name(in.op),
                                         dtype_name(nd.dtype)));
                break;
            case RV_CAST:
                if (!dtype_valid(in.dtype)) fail(RV_E_DTYPE, fmt("node %d: bad CAST dtype %d", i, in.dtype));
                nd.shape = S(0).shape;
                nd.dtype = in.dtype;
                break;
            case RV_ADD: case RV_MUL: case RV_CMPLT:
                if (S(0).shape != S(1).shape)
                    fail(RV_E_INVALID, fmt("node %d: %s of shapes %s and %s (broadcast with a VIEW first)", i,
                                           op_name(in.op), shape_str(S(0).shape).c_str(), shape_str(S(1).shape).c_str()));
                if (S(0).dtype != S(1).dtype)
                    fail(RV_E_DTYPE, fmt("node %d: %s of %s and %s", i, op_name(in.op), dtype_name(S(0).dtype),
                                         dtype_name(S(1).dtype)));
                nd.shape = S(0).shape;
                nd.dtype = in.op == RV_CMPLT ? RV_I8 : S(0).dtype;
                break;
            case RV_WHERE:
                if (S(0).shape != S(1).shape || S(1).shape != S(2).shape)
                    fail(RV_E_INVALID, fmt("node %d: WHERE operands differ in shape", i));
                if (S(1).dtype != S(2).dtype) fail(RV_E_DTYPE, fmt("node %d: WHERE branches differ in dtype", i));
                nd.shape = S(1).shape;
                nd.dtype = S(1).dtype;
                break;
            case RV_SUM: case RV_MAX: {
                const Shape& s = S(0).shape;
                if (s.size() < 32 && (in.reduce_axes >> s.size()) != 0)
                    fail(RV_E_INVALID, fmt("node %d: reduce axes 0x%x outside rank %zu", i, in.reduce_axes, s.size()));
                nd.shape = s;
                for (size_t d = 0; d < s.size(); ++d)
                    if (in.reduce_axes & (1u << d)) nd.shape[d] = 1;
                nd.dtype = S(0).dtype;
                nd.axes = in.reduce_axes;
                break;
            }
            case RV_CONTIGUOUS:
                nd.shape = S(0).shape;
                nd.dtype = S(0).dtype;
                break;
            case RV_GATHER: case RV_SCATTER: {
                // index (src 1) has the data's / base's shape but along the
                // axis; SCATTER's values (src 2) have the index's shape
                const char* nm = op_name(in.op);
                const Shape& d = S(0).shape;
                const Shape& ix = S(1).shape;
                uint32_t ax = in.reduce_axes;
                if (ax == 0 || (ax & (ax - 1)) != 0 || (d.size() < 32 && (ax >> d.size()) != 0))
                    fail(RV_E_INVALID, fmt("node %d: %s needs exactly one axis bit inside rank %zu, got 0x%x", i, nm,
                                           d.size(), ax));
                int a = 0;
                while (!((ax >> a) & 1u)) ++a;
                if (S(1).dtype != RV_I32)
                    fail(RV_E_DTYPE, fmt("node %d: %s index must be i32, got %s", i, nm, dtype_name(S(1).dtype)));
                bool ok = ix.size() == d.size();
                for (size_t k = 0; ok && k < d.size(); ++k) ok = (int)k == a || ix[k] == d[k];
                if (!ok)
                    fail(RV_E_INVALID, fmt("node %d: %s index shape %s must equal %s but along axis %d", i, nm,
                                           shape_str(ix).c_str(), shape_str(d).c_str(), a));
                nd.axis = a;
                if (in.op == RV_GATHER) {
                    if (in.buf != 0) fail(RV_E_INVALID, fmt("node %d: GATHER takes no flags", i));
                    nd.shape = ix;
                    nd.dtype = S(0).dtype;
                } else {
                    if (S(2).shape != ix)
                        fail(RV_E_INVALID, fmt("node %d: SCATTER values shape %s differs from the index's %s", i,
                                               shape_str(S(2).shape).c_str(), shape_str(ix).c_str()));
                    if (S(2).dtype != S(0).dtype)
                        fail(RV_E_DTYPE, fmt("node %d: SCATTER values %s into a %s base", i, dtype_name(S(2).dtype),
                                             dtype_name(S(0).dtype)));
                    if (in.buf != RV_SCATTER_ORDERED && in.buf != RV_SCATTER_ATOMIC)
                        fail(RV_E_INVALID, fmt("node %d: SCATTER mode %d", i, in.buf));
                    nd.atomic = in.buf == RV_SCATTER_ATOMIC;
                    const int dt = S(0).dtype;
                    if (nd.atomic && dt != RV_F32 && dt != RV_F64 && dt != RV_I32)
                        fail(RV_E_UNSUPPORTED_OP,
                             fmt("node %d: an atomic SCATTER of %s would also rewrite neighbouring cells of the word; "
                                 "atomic adds cover f32, f64 and i32 (the ordered mode covers every dtype)",
                                 i, dtype_name(dt)));
                    nd.shape = d;
                    nd.dtype = dt;
                }
                for (int64_t e : nd.shape)
                    if (e > (int64_t(1) << 31) - 1) fail(RV_E_INVALID, fmt("node %d: %s dims must fit in int32", i, nm));
                if (numel(ix) >= (int64_t(1) << 31))
                    fail(RV_E_INVALID, fmt("node %d: %s of 2^31 or more index cells", i, nm));
                break;
            }
            case RV_CUSTOM: {  // sdpa_fwd (the only CUSTOM kernel)
                const Shape &q = S(0).shape, &k = S(1).shape, &v = S(2).shape;
                for (int j = 0; j < 3; ++j)
                    if (S(j).dtype != RV_BF16) fail(RV_E_DTYPE, fmt("node %d: sdpa_fwd operands must be bf16", i));
                if (q.size() != 3 || k.size() != 3 || k != v || q[0] != k[0] || q[2] != k[2])
                    fail(RV_E_INVALID, fmt("node %d: sdpa_fwd needs q (H, Tq, D), k and v (H, Tk, D); got %s, %s, %s", i,
                                           shape_str(q).c_str(), shape_str(k).c_str(), shape_str(v).c_str()));
                if (q[2] != 32 && q[2] != 64 && q[2] != 128)
                    fail(RV_E_UNSUPPORTED_LAYOUT, fmt("node %d: sdpa_fwd head width %lld (32, 64 or 128)", i,
                                                      (long long)q[2]));
                if (q[1] < 1 || k[1] < 1 || q[0] < 1) fail(RV_E_INVALID, fmt("node %d: sdpa_fwd of an empty tensor", i));
                if (q[0] > 65535 || q[1] >= (int64_t(1) << 31) / q[2] || k[1] >= (int64_t(1) << 31) / k[2])
                    fail(RV_E_INVALID, fmt("node %d: sdpa_fwd too large", i));
                if ((in.reduce_axes & ~(RV_SDPA_CAUSAL | (0xffu << 16))) != 0)
                    fail(RV_E_INVALID, fmt("node %d: sdpa_fwd flags 0x%x", i, in.reduce_axes));
                nd.custom = in.buf;
                nd.cout = (int)((in.reduce_axes >> 16) & 0xff);
                nd.causal = (in.reduce_axes & RV_SDPA_CAUSAL) != 0;
                nd.cval = in.cval;
                // the kernel carries max(s) * scale as the running maximum of
                // the scaled scores and masks keys to -inf before scaling:
                // both hold only for a positive scale
                if (!(in.cval > 0.0) || in.cval == 1.0 / 0.0)
                    fail(RV_E_INVALID, fmt("node %d: sdpa_fwd scale must be finite and positive (got %g)", i, in.cval));
                if (nd.cout == 0) {
                    if (in.dtype != RV_F32 && in.dtype != RV_BF16)
                        fail(RV_E_DTYPE, fmt("node %d: sdpa_fwd output must be f32 or bf16", i));
                    nd.shape = q;
                    nd.dtype = in.dtype;
                } else if (nd.cout == 1) {
                    if (in.dtype != RV_F32) fail(RV_E_DTYPE, fmt("node %d: sdpa_fwd logsumexp is f32", i));
                    nd.shape = {q[0], q[1], 1};
                    nd.dtype = RV_F32;
                } else {
                    fail(RV_E_INVALID, fmt("node %d: sdpa_fwd has outputs 0 and 1, not %d", i, nd.cout));
                }
                break;
            }
        }
    }
    for (int k = 0; k < nout; ++k) {
        if (outputs[k] < 0 || outputs[k] >= n) fail(RV_E_INVALID, fmt("output %d names node %d", k, outputs[k]));
        g.outputs.push_back(outputs[k]);
    }
    g.users.assign(n, {});
    for (int i = 0; i < n; ++i)
        for (int k = 0; k < g.nodes[i].nsrc; ++k) g.users[g.nodes[i].src[k]].push_back(i);
    return g;
}

const char* kclass_name(KClass k) {
    switch (k) {
        case KClass::EW: return "EW";
        case KClass::ROW: return "ROW";
        case KClass::REDUCE: return "REDUCE";
        case KClass::MFMA: return "MFMA";
        case KClass::FOLD: return "FOLD";
        case KClass::ATTN: return "ATTN";
        case KClass::SCATTER: return "SCATTER";
        case KClass::SPLIT: return "SPLIT";
    }
    return "?";
}

}  // namespace rv
