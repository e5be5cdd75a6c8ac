// Scheduler: cuts the graph into kernels and builds each kernel's
// expression over its iteration domain.
//
// limn README, "Reading the schedule": elementwise work fuses into whatever
// consumes it, and a cut falls wherever a value has to exist in memory (a
// copy, an output, anything a View addresses). limn also cuts at every
// reduce; here a reduce is not cut when its consumers can keep the reduced
// value on chip:
//   ROW    reduces over the trailing dims of one row space, with their
//          elementwise producers and consumers (softmax, RMSNorm, LayerNorm):
//          a row is read once and stays in registers.
//   MFMA   SUM over k of CAST(bf16 A) * CAST(bf16 B) through stride-0 Views
//          (limn README's one-nest matmul; Luminal IR blog, "Naive Matrix
//          Multiplication"), with an elementwise epilogue on y and an
//          optional SUM of it over every dim.
//   REDUCE one thread per output cell, reduce loops run in order inside it
//          (limn README, "Backends": one point of the non-reduce dims per
//          thread, so results fold in the serial order).
//   EW     elementwise (incl. CONTIGUOUS of a permuted View = transpose).
// Values only differ from limn's per-reduce cuts in the order a fold
// associates its additions.
#include <algorithm>
#include <functional>
#include <map>
#include <set>

#include "graph.hpp"

namespace rv {

namespace {

using Map = std::vector<int>;  // node dim -> domain dim, or -1 (index 0)

constexpr int kRowMinLen = 128;  // shortest row handled by the ROW class

struct Ctx {
    Program& p;
    Graph& g;
    std::vector<char> mat;        // value exists in memory
    std::vector<std::vector<Loc>> loc;  // where (first entry is read by consumers)
};

// Compose a View over a value's storage with a map from the value's dims to
// the domain: the result addresses the same storage over the domain.
static Leaf compose_leaf(const rv_view& v, const Map& m, int rank, Loc loc, int dtype) {
    Leaf L;
    L.loc = loc;
    L.dtype = dtype;
    rv_view& o = L.v;
    o.ndim = rank;
    o.offset = v.offset;
    std::vector<int> hit(rank, 0);
    for (int d = 0; d < rank; ++d) {
        o.shape[d] = 0;  // filled by the caller (domain)
        o.strides[d] = 0;
        o.mask_lo[d] = 0;
        o.mask_hi[d] = INT64_MAX;
    }
    for (int d = 0; d < v.ndim; ++d) {
        int dd = m[d];
        if (dd < 0) {
            if (!(v.mask_lo[d] <= 0 && 0 < v.mask_hi[d])) L.zero = true;
            continue;
        }
        if (hit[dd]++) fail(RV_E_INVALID, "internal: two dims of one value map to one domain dim");
        o.strides[dd] = v.strides[d];
        o.mask_lo[dd] = v.mask_lo[d];
        o.mask_hi[dd] = v.mask_hi[d];
    }
    return L;
}

struct Builder {
    Ctx& c;
    Kernel& k;
    int root;
    enum Mode { EW, ROW, REDUCE, MFMA, FOLDK } mode;
    uint32_t rmask = 0;  // ROW/REDUCE: reduced domain dims
    int mfma_y = -1;     // MFMA: the contraction node
    int fold_red = -1;   // FOLDK: the split reduce whose folded partials this kernel reads
    std::map<std::pair<int, Map>, int> memo;
    std::map<std::pair<std::string, int>, int> leaf_memo;

    int rank() const { return (int)k.domain.size(); }

    int add(Ex e) {
        k.ex.push_back(e);
        return (int)k.ex.size() - 1;
    }

    int add_leaf(Leaf L) {
        for (int d = 0; d < rank(); ++d) {
            L.v.shape[d] = k.domain[d];
            L.v.mask_lo[d] = std::max<int64_t>(L.v.mask_lo[d], 0);
            L.v.mask_hi[d] = std::min<int64_t>(L.v.mask_hi[d], k.domain[d]);
            if (L.v.mask_hi[d] <= L.v.mask_lo[d]) L.zero = true;
        }
        std::string key = json_view(L.v) + fmt("|%d|%d|%d|%d", L.loc.kind, L.loc.index, L.dtype, (int)L.zero);
        auto it = leaf_memo.find({key, 0});
        if (it != leaf_memo.end()) return it->second;
        k.leaves.push_back(L);
        int id = (int)k.leaves.size() - 1;
        leaf_memo[{key, 0}] = id;
        return id;
    }

    int load(const rv_view& v, const Map& m, Loc loc, int dtype, int node) {
        Leaf L = compose_leaf(v, m, rank(), loc, dtype);
        Ex e;
        e.op = RV_BUFFER;
        e.dtype = dtype;
        e.leaf = add_leaf(L);
        e.node = node;
        return add(e);
    }

    int build(int i, const Map& m) {
        auto key = std::make_pair(i, m);
        auto it = memo.find(key);
        if (it != memo.end()) return it->second;
        int r = build_(i, m);
        memo[key] = r;
        return r;
    }

    int build_(int i, const Map& m) {
        const Node& nd = c.g.nodes[i];
        if (nd.op == RV_BUFFER)
            return load(view_contiguous(nd.shape), m, Loc{0, nd.slot}, nd.dtype, i);
        if (i != root && c.mat[i])
            return load(view_contiguous(nd.shape), m, c.loc[i][0], nd.dtype, i);
        switch (nd.op) {
            case RV_CONST: {
                Ex e;
                e.op = RV_CONST;
                e.dtype = nd.dtype;
                e.cval = nd.cval;
                e.node = i;
                return add(e);
            }
            case RV_VIEW: {
                int s = nd.src[0];
                const Node& sn = c.g.nodes[s];
                if (sn.op == RV_BUFFER) return load(nd.view, m, Loc{0, sn.slot}, sn.dtype, i);
                if (c.mat[s]) return load(nd.view, m, c.loc[s][0], sn.dtype, i);
                std::vector<int> sdv;
                if (!pure_broadcast(nd.view, sn.shape, &sdv))
                    fail(RV_E_INVALID, "internal: non-broadcast View of an unmaterialised value");
                Map sm(sn.shape.size(), -1);
                for (int dv = 0; dv < nd.view.ndim; ++dv)
                    if (sdv[dv] >= 0) sm[sdv[dv]] = m[dv];
                return build(s, sm);
            }
            case RV_CONTIGUOUS:
                return build(nd.src[0], m);
            case RV_SUM: case RV_MAX:
                return build_reduce(i, m);
            case RV_GATHER:
                return build_gather(i, m);
            default: break;
        }
        if (!is_elementwise(nd.op)) fail(RV_E_INVALID, fmt("internal: op %s in a kernel", op_name(nd.op)));
        Ex e;
        e.op = nd.op;
        e.dtype = nd.dtype;
        e.node = i;
        e.a = build(nd.src[0], m);
        if (nd.nsrc > 1) e.b = build(nd.src[1], m);
        if (nd.nsrc > 2) e.c = build(nd.src[2], m);
        return add(e);
    }

    // GATHER (a value in memory, so only its own elementwise kernel builds
    // it): the data is read where it lives, through its View with the
    // gathered axis left out; the index is fused.
    int build_gather(int i, const Map& m) {
        if (mode != EW) throw 1;
        const Node& nd = c.g.nodes[i];
        const int ds = nd.src[0];
        const Node& dn = c.g.nodes[ds];
        rv_view dv;
        Loc dl;
        if (dn.op == RV_BUFFER) {
            dv = view_contiguous(dn.shape);
            dl = Loc{0, dn.slot};
        } else if (c.mat[ds]) {
            dv = view_contiguous(dn.shape);
            dl = c.loc[ds][0];
        } else if (dn.op == RV_VIEW && (c.g.nodes[dn.src[0]].op == RV_BUFFER || c.mat[dn.src[0]])) {
            const Node& sn = c.g.nodes[dn.src[0]];
            dv = dn.view;
            dl = sn.op == RV_BUFFER ? Loc{0, sn.slot} : c.loc[dn.src[0]][0];
        } else {
            fail(RV_E_INVALID, "internal: GATHER data not in memory");
        }
        const int a = nd.axis;
        Ex e;
        e.op = RV_GATHER;
        e.dtype = nd.dtype;
        e.node = i;
        e.g_stride = dv.strides[a];
        e.g_lo = std::max<int64_t>(0, dv.mask_lo[a]);
        e.g_hi = std::min<int64_t>(dv.shape[a], dv.mask_hi[a]);
        rv_view v = dv;
        if (e.g_hi > e.g_lo) v.offset += e.g_lo * e.g_stride;
        v.strides[a] = 0;
        v.mask_lo[a] = 0;
        v.mask_hi[a] = 1;
        Map dm = m;
        dm[a] = -1;
        Leaf L = compose_leaf(v, dm, rank(), dl, dn.dtype);
        L.zero = L.zero || e.g_hi <= e.g_lo;
        e.leaf = add_leaf(L);
        e.a = build(nd.src[1], m);
        return add(e);
    }

    int build_reduce(int i, const Map& m) {
        const Node& nd = c.g.nodes[i];
        const Node& in = c.g.nodes[nd.src[0]];
        if (mode == MFMA && i == mfma_y) {
            Ex e;
            e.op = EX_MFMA_ACC;
            e.dtype = RV_F32;
            e.node = i;
            return add(e);
        }
        if (mode == FOLDK) {
            if (i != fold_red) throw 1;
            Ex e;
            e.op = EX_FOLD_ACC;
            e.dtype = nd.dtype;
            e.node = i;
            return add(e);
        }
        // ROW: the reduce must reduce exactly the domain's reduced dims of an
        // input laid over the whole domain; REDUCE: only the root reduces.
        if (!(mode == ROW || (mode == REDUCE && i == root))) throw 1;
        // (ROW reduces accumulate float32 for float32 and the half widths,
        // float64 for float64, and an exact wrapping total for ints)
        if (in.shape != k.domain) throw 1;
        uint32_t ax = 0;
        for (size_t d = 0; d < in.shape.size(); ++d)
            if ((nd.axes >> d) & 1u) ax |= (in.shape[d] == 1 ? 0u : (1u << d));
        if (ax != rmask) throw 1;
        for (size_t d = 0; d < nd.shape.size(); ++d) {
            bool red = (rmask >> d) & 1u;
            if (red ? m[d] != -1 : (m[d] != (int)d && nd.shape[d] != 1)) throw 1;
        }
        Map id(in.shape.size());
        for (size_t d = 0; d < id.size(); ++d) id[d] = (int)d;
        Ex e;
        e.op = nd.op;
        e.dtype = nd.dtype;
        e.node = i;
        e.axes = rmask;
        e.a = build(nd.src[0], id);
        e.stat = true;
        return add(e);
    }
};

// Reduces reachable from `root` without passing through a value in memory.
static void reach_reduces(Ctx& c, int root, std::set<int>& out, bool top_only) {
    std::set<int> seen;
    std::function<void(int)> go = [&](int i) {
        if (!seen.insert(i).second) return;
        const Node& nd = c.g.nodes[i];
        if (nd.op == RV_BUFFER) return;
        if (i != root && c.mat[i]) return;
        if (is_reduce(nd.op) && i != root) {
            out.insert(i);
            if (top_only) return;
        }
        if (nd.op == RV_VIEW) {
            int s = nd.src[0];
            if (c.g.nodes[s].op == RV_BUFFER || c.mat[s]) return;
            go(s);
            return;
        }
        for (int k = 0; k < nd.nsrc; ++k) go(nd.src[k]);
    };
    go(root);
}

static Map identity(size_t n) {
    Map m(n);
    for (size_t d = 0; d < n; ++d) m[d] = (int)d;
    return m;
}

static void add_stores(Ctx& c, Kernel& k, int root, int ex, const Map& m) {
    const Node& nd = c.g.nodes[root];
    for (const Loc& L : c.loc[root]) {
        Store s;
        s.ex = ex;
        s.loc = L;
        s.dtype = nd.dtype;
        s.node = root;
        Leaf lf = compose_leaf(view_contiguous(nd.shape), m, (int)k.domain.size(), L, nd.dtype);
        s.v = lf.v;
        for (size_t d = 0; d < k.domain.size(); ++d) {
            s.v.shape[d] = k.domain[d];
            s.v.mask_lo[d] = 0;
            s.v.mask_hi[d] = k.domain[d];
        }
        k.stores.push_back(s);
    }
}

// Map for a root of shape `shape` laid over `domain` (equal, or equal with
// the reduced dims set to 1).
static Map root_map(const Shape& shape, uint32_t rmask) {
    Map m(shape.size());
    for (size_t d = 0; d < shape.size(); ++d) m[d] = ((rmask >> d) & 1u) ? -1 : (int)d;
    return m;
}

static bool try_ew(Ctx& c, int root, Kernel& k) {
    std::set<int> red;
    reach_reduces(c, root, red, true);
    const Node& nd = c.g.nodes[root];
    if (!red.empty() || is_reduce(nd.op)) return false;
    k = Kernel{};
    k.cls = KClass::EW;
    k.domain = nd.shape;
    Builder b{c, k, root, Builder::EW};
    int e = b.build(root, identity(nd.shape.size()));
    add_stores(c, k, root, e, identity(nd.shape.size()));
    return true;
}

// CUSTOM sdpa_fwd: one kernel for a node and its siblings (same sources,
// scale and causal flag), reading q, k, v where they live (contiguous) and
// writing each sibling's output.
static bool same_sdpa(const Node& a, const Node& b) {
    return a.op == RV_CUSTOM && b.op == RV_CUSTOM && a.custom == b.custom && a.src[0] == b.src[0] &&
           a.src[1] == b.src[1] && a.src[2] == b.src[2] && a.cval == b.cval && a.causal == b.causal;
}

static void attn_kernel(Ctx& c, const std::vector<int>& nodes, Kernel& k) {
    const Node& nd = c.g.nodes[nodes[0]];
    k = Kernel{};
    k.cls = KClass::ATTN;
    const Shape& q = c.g.nodes[nd.src[0]].shape;
    k.domain = q;
    k.attn_scale = nd.cval;
    k.attn_causal = nd.causal;
    for (int j = 0; j < 3; ++j) {
        const Node& sn = c.g.nodes[nd.src[j]];
        Leaf L;
        L.loc = c.loc[nd.src[j]][0];
        L.dtype = sn.dtype;
        L.v = view_contiguous(sn.shape, 0);
        k.leaves.push_back(L);
    }
    for (int o : nodes) {
        const Node& on = c.g.nodes[o];
        for (const Loc& L : c.loc[o]) {
            Store st;
            st.ex = -1;
            st.loc = L;
            st.dtype = on.dtype;
            st.node = o;
            st.out_index = on.cout;
            st.v = view_contiguous(on.shape, 0);
            k.stores.push_back(st);
        }
    }
    // Keys are split into chunks of CK over workgroups when one workgroup
    // per 128-query block leaves the chip's workgroup slots empty (256 CUs,
    // each holding 4 of these workgroups at head width 32, 3 at 64, 2 at
    // 128: one wave per SIMD each), CK the smallest of 1024, 2048 and 4096
    // keeping the workgroups within twice the slots; under the causal mask
    // a block's chunks stop at its last key. Measured (one workgroup per
    // block against the chosen split): 6 x 8192 x 32 causal 1.4x faster,
    // non-causal 1.2x; 2 x 8192 x 128 causal 2.1x; 6 x 8192 x 128 causal
    // 1.27x; 4 x 4096 x 128 causal 1.8x; 16 x 2048 x 128 causal 5%.
    // RV_ATTN_CHUNK overrides (0: never split).
    const int64_t H = q[0], Tq = q[1], Tk = c.g.nodes[nd.src[1]].shape[1], D = q[2];
    const int64_t nqb0 = (Tq + 127) / 128, slots = 256 * (D == 32 ? 4 : D == 64 ? 3 : 2);
    auto workgroups = [&](int64_t ck) {
        int64_t n = 0;
        for (int64_t j = 0; j < nqb0; ++j) {
            const int64_t kend = k.attn_causal ? std::min(Tk, std::min(Tq, 128 * (j + 1))) : Tk;
            n += std::max<int64_t>(1, (kend + ck - 1) / ck);
        }
        return n * H;
    };
    int64_t CKd = 0;
    if (H * nqb0 < slots)
        for (int64_t ck : {1024, 2048, 4096})
            if (workgroups(ck) <= 2 * slots || ck == 4096) {
                CKd = ck;
                break;
            }
    int64_t CK = env_int("RV_ATTN_CHUNK", (int)CKd);
    if (CK < 0) fail(RV_E_INVALID, "RV_ATTN_CHUNK must be 0 or positive");
    if (CK > 0) {
        CK = (CK + 127) / 128 * 128;
        const int64_t nqb = (Tq + 127) / 128;
        std::vector<unsigned> map;
        int64_t cmax = 1;
        for (int64_t j = nqb - 1; j >= 0; --j) {
            const int64_t kend = k.attn_causal ? std::min(Tk, std::min(Tq, 128 * (j + 1))) : Tk;
            const int64_t nch = std::max<int64_t>(1, (kend + CK - 1) / CK);
            cmax = std::max(cmax, nch);
            for (int64_t ch = 0; ch < nch; ++ch) map.push_back((unsigned)((j << 16) | ch));
        }
        if (cmax > 1 && cmax < 65536 && nqb < 65536 && (int64_t)map.size() <= 65535) {
            k.attn_chunk = CK;
            k.attn_cmax = (int)cmax;
            k.attn_map = map;
            k.attn_reg_o = (int)c.p.regions.size();
            c.p.regions.push_back(Region{0, (size_t)(H * nqb * cmax * 128 * D * 4)});
            k.attn_reg_ml = (int)c.p.regions.size();
            c.p.regions.push_back(Region{0, (size_t)(H * nqb * cmax * 128 * 2 * 4)});
        }
    }
}

// Row space of a reduce: (input shape, reduced dims) with every reduced
// non-size-1 dim after every kept non-size-1 dim.
static bool row_space(const Node& r, const Node& in, uint32_t* rmask) {
    uint32_t ax = 0;
    int last_kept = -1, first_red = 1 << 20;
    for (size_t d = 0; d < in.shape.size(); ++d) {
        if (in.shape[d] == 1) continue;
        if ((r.axes >> d) & 1u) {
            ax |= 1u << d;
            first_red = std::min(first_red, (int)d);
        } else {
            last_kept = (int)d;
        }
    }
    if (ax == 0 || last_kept > first_red) return false;
    *rmask = ax;
    return true;
}

static bool try_row(Ctx& c, int root, Kernel& k) {
    std::set<int> red;
    reach_reduces(c, root, red, false);
    const Node& rn = c.g.nodes[root];
    if (is_reduce(rn.op)) red.insert(root);
    if (red.empty()) return false;
    int r0 = *red.begin();
    const Node& in0 = c.g.nodes[c.g.nodes[r0].src[0]];
    uint32_t rmask;
    if (!row_space(c.g.nodes[r0], in0, &rmask)) return false;
    int64_t n = 1;
    for (size_t d = 0; d < in0.shape.size(); ++d)
        if ((rmask >> d) & 1u) n *= in0.shape[d];
    if (n < kRowMinLen) return false;
    // the root is the full row space or its per-row statistics
    Shape stat = in0.shape;
    for (size_t d = 0; d < stat.size(); ++d)
        if ((rmask >> d) & 1u) stat[d] = 1;
    if (rn.shape != in0.shape && rn.shape != stat) return false;
    Kernel kk;
    kk.cls = KClass::ROW;
    kk.domain = in0.shape;
    kk.rdims = rmask;
    Builder b{c, kk, root, Builder::ROW};
    b.rmask = rmask;
    Map m = rn.shape == in0.shape ? identity(rn.shape.size()) : root_map(rn.shape, rmask);
    try {
        int e = b.build(root, m);
        add_stores(c, kk, root, e, m);
    } catch (int) {
        return false;
    }
    k = kk;
    return true;
}

static bool try_reduce_cells(Ctx& c, int root, Kernel& k) {
    const Node& rn = c.g.nodes[root];
    if (!is_reduce(rn.op)) return false;
    std::set<int> red;
    reach_reduces(c, root, red, true);
    if (!red.empty()) return false;
    const Node& in = c.g.nodes[rn.src[0]];
    uint32_t rmask = 0;
    for (size_t d = 0; d < in.shape.size(); ++d)
        if (((rn.axes >> d) & 1u) && in.shape[d] != 1) rmask |= 1u << d;
    Kernel kk;
    kk.cls = KClass::REDUCE;
    kk.domain = in.shape;
    kk.rdims = rmask;
    Builder b{c, kk, root, Builder::REDUCE};
    b.rmask = rmask;
    Map m = root_map(rn.shape, rmask);
    try {
        int e = b.build(root, m);
        add_stores(c, kk, root, e, m);
    } catch (int) {
        return false;
    }
    k = kk;
    return true;
}

// ---- split reduce ----------------------------------------------------------
//
// limn README, "Backends": a long reduce over few cells splits into strided
// partial totals and a fold. A region whose only reduce has few output cells
// for the length it reduces would leave most of the chip idle as one
// workgroup per row (ROW) or one lane per cell (REDUCE); it becomes a SPLIT
// kernel (each workgroup folds one piece of the reduce range for its cells,
// in a fixed order, into a partials region) and a FOLD kernel (the pieces of
// each cell folded in piece order, then the region's elementwise tail on the
// result). No atomics: two runs give the same bits.

// Output cells and reduce length of reduce node r.
static void reduce_extent(const Ctx& c, int r, int64_t* cells, int64_t* len) {
    const Node& R = c.g.nodes[r];
    const Node& in = c.g.nodes[R.src[0]];
    *cells = numel(R.shape);
    *len = *cells > 0 ? numel(in.shape) / *cells : 0;
}

// Whether a reduce of `cells` outputs over `len` terms each pays for the
// extra launch: enough work in total, and the one-kernel plans would start
// fewer workgroups than the chip has CUs (256): ROW takes a workgroup per
// row (long rows), REDUCE a workgroup per 256 cells.
static bool split_pays(const Ctx& c, int r, int64_t cells, int64_t len) {
    if (cells <= 0 || len < 512 || cells * len < ((int64_t)1 << 20)) return false;
    uint32_t rm;
    const Node& R = c.g.nodes[r];
    const bool rowlike = row_space(R, c.g.nodes[R.src[0]], &rm) && len >= kRowMinLen;
    if (rowlike) return cells < 256 && len >= 8192;
    return (cells + 255) / 256 < 256;
}

static bool try_split(Ctx& c, int root, std::vector<Kernel>& out) {
    if (env_int("RV_SPLIT", 1) == 0) return false;
    std::set<int> red;
    reach_reduces(c, root, red, false);
    const Node& rn = c.g.nodes[root];
    int r;
    if (is_reduce(rn.op)) {
        if (!red.empty()) return false;
        r = root;
    } else {
        if (red.size() != 1) return false;
        r = *red.begin();
        if (rn.shape != c.g.nodes[r].shape) return false;
    }
    const Node& R = c.g.nodes[r];
    const Node& in = c.g.nodes[R.src[0]];
    int64_t cells, len;
    reduce_extent(c, r, &cells, &len);
    if (!split_pays(c, r, cells, len)) return false;
    uint32_t rmask = 0;
    for (size_t d = 0; d < in.shape.size(); ++d)
        if (((R.axes >> d) & 1u) && in.shape[d] != 1) rmask |= 1u << d;
    if (!rmask) return false;
    Kernel kp;
    kp.cls = KClass::SPLIT;
    kp.domain = in.shape;
    kp.rdims = rmask;
    kp.red_op = R.op;
    kp.red_dtype = R.dtype;
    Kernel kf;
    kf.cls = KClass::FOLD;
    kf.domain = R.shape;
    kf.red_op = R.op;
    kf.red_dtype = R.dtype;
    try {
        Builder b{c, kp, r, Builder::REDUCE};
        b.rmask = rmask;
        b.build(r, root_map(R.shape, rmask));
        Builder bf{c, kf, root, Builder::FOLDK};
        bf.fold_red = r;
        int e = bf.build(root, identity(R.shape.size()));
        add_stores(c, kf, root, e, identity(R.shape.size()));
    } catch (int) {
        return false;
    }
    kp.partials_region = (int)c.p.regions.size();
    c.p.regions.push_back(Region{});  // sized when the pieces are planned
    kf.fold_src_region = kp.partials_region;
    out.push_back(kp);
    out.push_back(kf);
    return true;
}

// A region with several reduces over few long rows (a softmax of a handful
// of 1 MB rows): the ROW plan would run one workgroup per row. Its topmost
// reduces are cut instead, so each becomes a split reduce.
static bool cut_for_split(Ctx& c, int root, std::set<int>* top) {
    if (env_int("RV_SPLIT", 1) == 0) return false;
    std::set<int> red;
    reach_reduces(c, root, red, false);
    if (is_reduce(c.g.nodes[root].op)) red.insert(root);
    if (red.size() < 2) return false;
    for (int r : red) {
        int64_t cells, len;
        reduce_extent(c, r, &cells, &len);
        if (!split_pays(c, r, cells, len)) return false;
    }
    reach_reduces(c, root, *top, true);
    return !top->empty();
}

// ---- MFMA ----------------------------------------------------------------

// Strips CASTs to f32 and returns the leaf-producing node (a bf16 BUFFER, or
// a chain of VIEWs over one or over a value in memory, which the builder
// composes into one View) under a f32 CAST, or -1.
static int bf16_operand(Ctx& c, int i) {
    const Node& nd = c.g.nodes[i];
    if (nd.op != RV_CAST || nd.dtype != RV_F32 || c.mat[i]) return -1;
    int s = nd.src[0];
    const Node& sn = c.g.nodes[s];
    if (sn.dtype != RV_BF16) return -1;
    if (sn.op == RV_BUFFER) return s;
    for (int v = s; c.g.nodes[v].op == RV_VIEW && !c.mat[v];) {
        const int src = c.g.nodes[v].src[0];
        if (c.g.nodes[src].op == RV_BUFFER || c.mat[src]) return s;
        v = src;
    }
    return -1;
}

static bool is_contraction(Ctx& c, int y) {
    const Node& yn = c.g.nodes[y];
    if (yn.op != RV_SUM) return false;
    const Node& mul = c.g.nodes[yn.src[0]];
    if (mul.op != RV_MUL || mul.dtype != RV_F32 || c.mat[yn.src[0]]) return false;
    if (mul.shape.size() != 3 || yn.axes != 4u) return false;
    return bf16_operand(c, mul.src[0]) >= 0 && bf16_operand(c, mul.src[1]) >= 0;
}

// A zero-padded copy of a contraction operand into workspace region `region`:
// `rows` x `cols` row-major, cell (r, c) = the operand at domain dims
// (dr, dc) = (r, c) when r < R and c < C (and inside its View's mask), else
// zero. An elementwise kernel of its own (a transposing copy when the
// operand is stored the other way round).
static Kernel operand_copy(const Leaf& L, int dr, int dc, int64_t rows, int64_t cols, int64_t R, int64_t C,
                           int region) {
    Kernel kc;
    kc.cls = KClass::EW;
    kc.domain = Shape{rows, cols};
    Leaf s;
    s.loc = L.loc;
    s.dtype = RV_BF16;
    s.zero = L.zero;
    s.v.ndim = 2;
    s.v.offset = L.v.offset;
    const int ds[2] = {dr, dc};
    const int64_t ext[2] = {R, C}, sz[2] = {rows, cols};
    for (int j = 0; j < 2; ++j) {
        s.v.shape[j] = sz[j];
        s.v.strides[j] = L.v.strides[ds[j]];
        s.v.mask_lo[j] = std::max<int64_t>(0, L.v.mask_lo[ds[j]]);
        s.v.mask_hi[j] = std::min<int64_t>(ext[j], L.v.mask_hi[ds[j]]);
        if (s.v.mask_hi[j] <= s.v.mask_lo[j]) s.zero = true;
    }
    kc.leaves.push_back(s);
    Ex e;
    e.op = RV_BUFFER;
    e.dtype = RV_BF16;
    e.leaf = 0;
    kc.ex.push_back(e);
    Store st;
    st.ex = 0;
    st.loc = Loc{2, region};
    st.dtype = RV_BF16;
    st.v = view_contiguous(Shape{rows, cols});
    kc.stores.push_back(st);
    return kc;
}

// Operands of the contraction kernel. One is read in place when the kernel's
// copies can address it directly: contiguous along k (A; B along k or n),
// 16-byte aligned rows, unmasked, at least one 256-wide tile along its
// output dim, and K a multiple of the 32-deep k-tile. Any other operand
// (ragged K, a narrow M or N, a transposed, padded, windowed or unaligned
// View) is first copied into workspace, zero-padded to those extents, by an
// elementwise kernel; every bf16 contraction thus runs on the matrix cores.
// The copies are appended to `out`; the kernel's leaves and extents are
// rewritten to read them.
static void mfma_operands(Ctx& c, Kernel& k, std::vector<Kernel>& out) {
    const int64_t M = k.domain[0], N = k.domain[1], K = k.domain[2];
    const int64_t KS = kMfmaKStep;
    const int64_t Kp = (K + KS - 1) / KS * KS, lim = (int64_t)1 << 27;
    const Leaf A = k.leaves[k.mfma_a], B = k.leaves[k.mfma_b];
    auto unmasked = [](const Leaf& L) {
        if (L.zero) return false;
        for (int d = 0; d < 3; ++d)
            if (L.v.mask_lo[d] != 0 || L.v.mask_hi[d] != L.v.shape[d]) return false;
        return true;
    };
    const rv_view &a = A.v, &b = B.v;
    const bool a_direct = K % KS == 0 && unmasked(A) && M >= 256 && a.strides[2] == 1 && a.offset % 8 == 0 &&
                          a.strides[0] % 8 == 0 && a.strides[0] < lim;
    const bool kn = b.strides[1] == 1;
    const bool b_direct = K % KS == 0 && unmasked(B) && N >= 256 && b.offset % 8 == 0 &&
                          (kn ? (b.strides[2] % 8 == 0 && N % 8 == 0 && b.strides[2] < lim)
                              : (b.strides[2] == 1 && b.strides[1] % 8 == 0 && b.strides[1] < lim));
    int64_t Me = M, Ne = N;
    auto region = [&](int64_t elems) {
        c.p.regions.push_back(Region{0, (size_t)elems * 2});
        return (int)c.p.regions.size() - 1;
    };
    if (!a_direct) {
        Me = std::max<int64_t>(M, 256);
        const int r = region(Me * Kp);
        out.push_back(operand_copy(A, 0, 2, Me, Kp, M, K, r));
        Leaf L;
        L.loc = Loc{2, r};
        L.dtype = RV_BF16;
        L.v = view_contiguous(k.domain);
        L.v.strides[0] = Kp;
        L.v.strides[1] = 0;
        L.v.strides[2] = 1;
        k.leaves.push_back(L);
        k.mfma_a = (int)k.leaves.size() - 1;
        k.mfma_copied[0] = true;
    }
    if (!b_direct) {
        Leaf L;
        L.dtype = RV_BF16;
        L.v = view_contiguous(k.domain);
        L.v.strides[0] = 0;
        if (b.strides[2] == 1) {  // stored along k: copied as [n][k]
            Ne = std::max<int64_t>(N, 256);
            const int r = region(Ne * Kp);
            out.push_back(operand_copy(B, 1, 2, Ne, Kp, N, K, r));
            L.loc = Loc{2, r};
            L.v.strides[1] = Kp;
            L.v.strides[2] = 1;
        } else {  // as [k][n], rows padded to whole 16-byte chunks
            Ne = std::max<int64_t>((N + 7) / 8 * 8, 256);
            const int r = region(Kp * Ne);
            out.push_back(operand_copy(B, 2, 1, Kp, Ne, K, N, r));
            L.loc = Loc{2, r};
            L.v.strides[1] = 1;
            L.v.strides[2] = Ne;
        }
        k.leaves.push_back(L);
        k.mfma_b = (int)k.leaves.size() - 1;
        k.mfma_copied[1] = true;
    }
    k.mfma_ext[0] = Me;
    k.mfma_ext[1] = Ne;
    k.mfma_ext[2] = Kp;
}

// Slices over k for a contraction whose output tiles leave most of the 256
// CUs idle: S slices put S x tiles workgroups on the chip, at the cost of S
// float32 accumulator planes written and read back. The count minimises a
// time estimate: one workgroup's k-loop at a measured per-CU rate, plus, once
// split, the second kernel's launch and the planes' traffic. Planes stay
// within 32 MiB unless RV_GEMM_SPLITK forces a count (1: no split).
static int mfma_split_count(const Kernel& k) {
    const int64_t M = k.domain[0], N = k.domain[1];
    const int64_t Me = k.mfma_ext[0], Ne = k.mfma_ext[1], Ke = k.mfma_ext[2];
    const int64_t tiles = ((Me + 255) / 256) * ((Ne + 255) / 256);
    auto fits = [&](int64_t S) { return tiles * S <= 256 && Ke % (kMfmaKStep * S) == 0 && Ke / S >= 4 * kMfmaKStep; };
    const int forced = env_int("RV_GEMM_SPLITK", 0);
    if (forced >= 1) return forced > 1 && (forced & (forced - 1)) == 0 && fits(forced) ? forced : 1;
    auto fits_ws = [&](int64_t S) { return fits(S) && S * M * N * 4 <= ((int64_t)32 << 20); };
    const double cu_flops = 7e12, plane_bw = 5e12, launch_us = 3.0;
    auto est_us = [&](int64_t S) {
        const double loop = 2.0 * 256 * 256 * (double)(Ke / S) / cu_flops * 1e6;
        return S == 1 ? loop : loop + launch_us + (double)(S * M * N * 8) / plane_bw * 1e6;
    };
    int64_t best = 1;
    for (int64_t S = 2; fits_ws(S); S *= 2)
        if (est_us(S) < est_us(best)) best = S;
    return (int)best;
}

static bool try_mfma(Ctx& c, int root, std::vector<Kernel>& out, int& partial_region) {
    const Node& rn = c.g.nodes[root];
    int y = -1, epi_root = -1;
    bool partial = false;
    auto single_contraction_below = [&](int top) -> int {
        std::set<int> red;
        reach_reduces(c, top, red, false);
        if (red.size() != 1) return -1;
        int cand = *red.begin();
        return is_contraction(c, cand) ? cand : -1;
    };
    if (is_contraction(c, root)) {
        y = root;
        epi_root = root;
    } else if (rn.op == RV_SUM) {
        const Node& in = c.g.nodes[rn.src[0]];
        bool all = true;
        for (size_t d = 0; d < in.shape.size(); ++d)
            if (in.shape[d] != 1 && !((rn.axes >> d) & 1u)) all = false;
        if (!all || c.mat[rn.src[0]]) return false;
        y = single_contraction_below(rn.src[0]);
        if (y < 0 || in.shape != c.g.nodes[y].shape) return false;
        epi_root = rn.src[0];
        partial = true;
    } else if (!is_reduce(rn.op)) {
        y = single_contraction_below(root);
        if (y < 0 || rn.shape != c.g.nodes[y].shape) return false;
        epi_root = root;
    } else {
        return false;
    }
    const Node& yn = c.g.nodes[y];
    const Node& mul = c.g.nodes[yn.src[0]];
    Kernel k;
    k.cls = KClass::MFMA;
    k.domain = mul.shape;  // (M, N, K)
    k.rdims = 4u;
    Builder b{c, k, root, Builder::MFMA};
    b.mfma_y = y;
    b.rmask = 4u;
    // operand leaves over (M, N, K)
    Map id3 = identity(3);
    int ea = b.build(bf16_operand(c, mul.src[0]), id3);
    int eb = b.build(bf16_operand(c, mul.src[1]), id3);
    int la = k.ex[ea].leaf, lb = k.ex[eb].leaf;
    auto sv = [&](int l, int d) { return k.leaves[l].v.strides[d]; };
    // A walks (m, k) with n-stride 0; B walks (n, k) with m-stride 0
    if (sv(la, 1) != 0 || sv(lb, 0) != 0) std::swap(la, lb);
    if (sv(la, 1) != 0 || sv(lb, 0) != 0) return false;
    const int64_t M = k.domain[0], N = k.domain[1], K = k.domain[2];
    // an empty contraction has nothing for the matrix cores: the other
    // classes write its identity
    if (M == 0 || N == 0 || K == 0) return false;
    if (M >= ((int64_t)1 << 30) || N >= ((int64_t)1 << 30) || K >= ((int64_t)1 << 30))
        fail(RV_E_UNSUPPORTED_LAYOUT, fmt("contraction (%lld, %lld, %lld): extents of 2^30 or more",
                                          (long long)M, (long long)N, (long long)K));
    k.mfma_a = la;
    k.mfma_b = lb;
    // the epilogue over (M, N, 1): built on the contraction's output map
    Map ym = root_map(yn.shape, 4u);
    int e;
    try {
        e = b.build(epi_root, ym);
    } catch (int) {
        return false;
    }
    k.mfma_y = y;
    // epilogue leaves must not walk k
    for (size_t l = 0; l < k.leaves.size(); ++l)
        if ((int)l != la && (int)l != lb && k.leaves[l].v.strides[2] != 0) return false;
    mfma_operands(c, k, out);
    const int S = mfma_split_count(k);
    if (S > 1) {
        // the slice kernel (operands in, raw planes out), then this one
        // folding the planes into the epilogue
        Kernel ks = k;
        ks.mfma_split = S;
        ks.slices_region = (int)c.p.regions.size();
        c.p.regions.push_back(Region{0, (size_t)(S * ((M * N + 63) / 64 * 64)) * 4});
        out.push_back(ks);
        k.mfma_split = S;
        k.mfma_slices = true;
        k.slices_region = ks.slices_region;
    }
    if (partial) {
        k.mfma_partial = true;
        Store s;
        s.ex = e;
        s.dtype = RV_F32;
        s.node = root;
        k.stores.push_back(s);  // target set in lower() (partials region)
        partial_region = (int)c.p.regions.size();
        c.p.regions.push_back(Region{});
        k.partials_region = partial_region;
    } else {
        add_stores(c, k, root, e, ym);
    }
    out.push_back(k);
    if (partial) {
        Kernel f;
        f.cls = KClass::FOLD;
        f.domain = Shape{1};
        f.fold_src_region = partial_region;
        Ex acc;
        acc.op = RV_SUM;
        acc.dtype = rn.dtype;
        acc.node = root;
        f.ex.push_back(acc);
        add_stores(c, f, root, 0, Map(rn.shape.size(), -1));
        out.push_back(f);
    }
    return true;
}

// ---- SCATTER ---------------------------------------------------------------

static int bit_width(uint64_t x) {
    int b = 0;
    while (x) {
        ++b;
        x >>= 1;
    }
    return b;
}

// The kernels of one SCATTER node. Ordered: keys, stable radix passes, and
// a fold that writes every output cell once (the base, plus the cell's run
// of values in index order). Atomic: a fill (out = base, elementwise) and
// one atomic-add kernel. Then copies to any further output locations.
// Returns false (after marking what must exist in memory first) when a
// source cannot be fused.
static bool scatter_kernels(Ctx& c, int i, std::vector<Kernel>& out, std::vector<char>& need) {
    const Node& nd = c.g.nodes[i];
    const Shape& osh = nd.shape;
    const Shape& ish = c.g.nodes[nd.src[1]].shape;
    const std::vector<Loc> all = c.loc[i];
    const Loc target = all[0];
    const bool ordered = !nd.atomic && numel(ish) > 0;
    std::vector<Kernel> ks;
    if (!ordered) {  // fill
        Kernel f;
        f.cls = KClass::EW;
        f.domain = osh;
        Builder b{c, f, i, Builder::EW};
        c.loc[i] = {target};
        try {
            int e = b.build(nd.src[0], identity(osh.size()));
            add_stores(c, f, i, e, identity(osh.size()));
        } catch (int) {
            c.loc[i] = all;
            need[nd.src[0]] = 1;
            return false;
        }
        c.loc[i] = all;
        ks.push_back(f);
    }
    Kernel k;
    k.cls = KClass::SCATTER;
    k.domain = ish;
    Builder b{c, k, i, Builder::EW};
    for (int j = 1; j <= 2; ++j) {
        try {
            int e = b.build(nd.src[j], identity(ish.size()));
            (j == 1 ? k.sc_index : k.sc_values) = e;
        } catch (int) {
            need[nd.src[j]] = 1;
            return false;
        }
    }
    if (ordered) {  // the base, over the output's shape (its own memo: a
                    // source shared with the values is another domain here)
        k.domain = osh;
        Builder bb{c, k, i, Builder::EW};
        try {
            k.sc_base = bb.build(nd.src[0], identity(osh.size()));
        } catch (int) {
            need[nd.src[0]] = 1;
            return false;
        }
        k.domain = ish;
    }
    k.sc_axis = nd.axis;
    k.sc_out = target;
    k.sc_out_shape = osh;
    k.sc_dtype = nd.dtype;
    int64_t cells = 1, keys = osh[nd.axis];
    for (size_t d = 0; d < ish.size(); ++d) {
        const bool carried = (int)d != nd.axis && ish[d] > 1 && ex_invariant(k, k.sc_index, (int)d);
        if (carried) {
            k.sc_fdims |= 1u << d;
            continue;
        }
        cells *= ish[d];
        if ((int)d != nd.axis) keys *= ish[d];
    }
    k.sc_cells = cells;
    k.sc_keys_n = keys;
    if (numel(ish) > 0) {
        if (nd.atomic) {
            k.sc_part = "atomic";
            ks.push_back(k);
        } else {
            // keys, sorted positions and cell ids travel as 32-bit words whose
            // bit 31 flags a dropped cell, and the run bounds are read as int
            if (keys >= (int64_t(1) << 31))
                fail(RV_E_INVALID, fmt("SCATTER into %s: %lld target keys (2^31 or more)",
                                       shape_str(osh).c_str(), (long long)keys));
            const int passes = std::max(1, (bit_width((uint64_t)keys - 1) + 7) / 8);
            const int64_t nb = (cells + 2047) / 2048;
            auto region = [&](int64_t bytes) {
                c.p.regions.push_back(Region{0, (size_t)bytes});
                return (int)c.p.regions.size() - 1;
            };
            for (int q = 0; q < 2; ++q) {
                k.sc_reg_keys[q] = region(cells * 4);
                k.sc_reg_vals[q] = region(cells * 4);
            }
            if (nb > kScanInline) k.sc_reg_counts = region((256 * nb + 256) * 4);
            k.sc_reg_bounds = region((keys + 1) * 4);
            k.sc_passes = passes;
            // with the digit counts done inside the moves (few tiles), the
            // first move computes its keys from the index itself
            const bool fuse = nb <= kScanInline;
            if (!fuse) {
                Kernel kk = k;
                kk.sc_part = "keys";
                ks.push_back(kk);
            }
            for (int q = 0; q < passes; ++q)
                for (const char* part : {"hist", "scan", "move"}) {
                    if (std::string(part) != "move" && nb <= kScanInline) continue;
                    Kernel r = k;
                    if (fuse && q == 0) {
                        r.sc_values = r.sc_base = -1;
                        r.sc_fused_keys = true;
                    } else {
                        r.leaves.clear();
                        r.ex.clear();
                        r.sc_index = r.sc_values = r.sc_base = -1;
                    }
                    r.sc_part = part;
                    r.sc_pass = q;
                    ks.push_back(r);
                }
            Kernel bd = k;
            bd.leaves.clear();
            bd.ex.clear();
            bd.sc_index = bd.sc_values = bd.sc_base = -1;
            bd.sc_part = "bounds";
            ks.push_back(bd);
            Kernel fo = k;
            fo.sc_part = "fold";
            ks.push_back(fo);
        }
    }
    // further locations of the same output: copies of the first
    if (all.size() > 1) {
        Kernel kc;
        kc.cls = KClass::EW;
        kc.domain = osh;
        Builder bc{c, kc, i, Builder::EW};
        int e = bc.load(view_contiguous(osh), identity(osh.size()), target, nd.dtype, i);
        c.loc[i] = std::vector<Loc>(all.begin() + 1, all.end());
        add_stores(c, kc, i, e, identity(osh.size()));
        c.loc[i] = all;
        ks.push_back(kc);
    }
    for (auto& x : ks) out.push_back(x);
    return true;
}

}  // namespace

bool ex_invariant(const Kernel& k, int e, int d) {
    if (e < 0) return true;
    const Ex& x = k.ex[e];
    auto leaf_inv = [&](int l) {
        const Leaf& L = k.leaves[l];
        return L.zero || (L.v.strides[d] == 0 && L.v.mask_lo[d] <= 0 && L.v.mask_hi[d] >= L.v.shape[d]);
    };
    if (x.op == RV_BUFFER) return leaf_inv(x.leaf);
    if (x.op == RV_CONST) return true;
    if (x.op == RV_GATHER && !leaf_inv(x.leaf)) return false;
    return ex_invariant(k, x.a, d) && ex_invariant(k, x.b, d) && ex_invariant(k, x.c, d);
}

void schedule(Program& p) {
    Graph& g = p.g;
    const int n = (int)g.nodes.size();
    // a View of a View reads the inner View's source directly when the two
    // compose into one View (nodes are in order, so chains collapse whole);
    // otherwise the inner value is materialised below
    for (int i = 0; i < n; ++i) {
        Node& nd = g.nodes[i];
        if (nd.op != RV_VIEW) continue;
        const Node& s = g.nodes[nd.src[0]];
        if (s.op != RV_VIEW) continue;
        rv_view c;
        if (view_compose(s.view, nd.view, &c)) {
            nd.src[0] = s.src[0];
            nd.view = c;
        }
    }
    Ctx c{p, g, std::vector<char>(n, 0), std::vector<std::vector<Loc>>(n)};
    for (int i = 0; i < n; ++i)
        if (g.nodes[i].op == RV_BUFFER) {
            c.mat[i] = 1;
            c.loc[i].push_back(Loc{0, g.nodes[i].slot});
        }
    std::vector<char> is_out(n, 0);
    for (size_t k = 0; k < g.outputs.size(); ++k) is_out[g.outputs[k]] = 1;
    // values that must exist in memory
    std::vector<char> need(n, 0);
    for (int i = 0; i < n; ++i) {
        const Node& nd = g.nodes[i];
        if (is_out[i] || nd.op == RV_CONTIGUOUS || nd.op == RV_GATHER || nd.op == RV_SCATTER) need[i] = 1;
        if (nd.op == RV_GATHER) {  // the data is read where it lives
            const int ds = nd.src[0];
            const Node& dn = g.nodes[ds];
            if (dn.op == RV_VIEW) {
                if (g.nodes[dn.src[0]].op != RV_BUFFER) need[dn.src[0]] = 1;
            } else if (dn.op != RV_BUFFER) {
                need[ds] = 1;
            }
        }
        if (nd.op == RV_CUSTOM)  // the kernel reads its operands from memory
            for (int j = 0; j < nd.nsrc; ++j)
                if (g.nodes[nd.src[j]].op != RV_BUFFER) need[nd.src[j]] = 1;
        if (nd.op == RV_VIEW) {
            int s = nd.src[0];
            const Node& sn = g.nodes[s];
            if (sn.op == RV_BUFFER) continue;
            if (!pure_broadcast(nd.view, sn.shape, nullptr)) need[s] = 1;
        }
    }
    std::vector<Kernel> kernels;
    // Fixed point: a root whose region cannot be one kernel has its topmost
    // reduces cut (they get their own kernels) and is planned again.
    for (int iter = 0; iter < 4 * n + 4; ++iter) {
        for (int i = 0; i < n; ++i) c.mat[i] = (g.nodes[i].op == RV_BUFFER) || need[i];
        kernels.clear();
        p.regions.clear();
        bool again = false;
        std::vector<char> covered(n, 0);  // CUSTOM siblings written by an earlier node's kernel
        auto place = [&](int i) {  // location of the value
            c.loc[i].clear();
            for (size_t k = 0; k < g.outputs.size(); ++k)
                if (g.outputs[k] == i) c.loc[i].push_back(Loc{1, (int)k});
            if (c.loc[i].empty()) {
                c.loc[i].push_back(Loc{2, (int)p.regions.size()});
                p.regions.push_back(Region{0, (size_t)numel(g.nodes[i].shape) * dtype_size(g.nodes[i].dtype)});
            }
        };
        for (int i = 0; i < n && !again; ++i) {
            if (!need[i] || g.nodes[i].op == RV_BUFFER || covered[i]) continue;
            place(i);
            Kernel k;
            int preg = -1;
            std::vector<Kernel> mk;
            if (g.nodes[i].op == RV_CUSTOM) {
                std::vector<int> sib{i};
                for (int j = i + 1; j < n; ++j)
                    if (need[j] && same_sdpa(g.nodes[i], g.nodes[j])) {
                        place(j);
                        covered[j] = 1;
                        sib.push_back(j);
                    }
                attn_kernel(c, sib, k);
                kernels.push_back(k);
                if (k.attn_chunk > 0) {  // fold the chunk partials
                    Kernel mk = k;
                    mk.attn_merge = true;
                    mk.attn_map.clear();
                    kernels.push_back(mk);
                }
            } else if (g.nodes[i].op == RV_SCATTER) {
                if (!scatter_kernels(c, i, kernels, need)) again = true;
            } else if (try_ew(c, i, k)) {
                kernels.push_back(k);
            } else if (try_mfma(c, i, mk, preg)) {
                for (auto& x : mk) kernels.push_back(x);
            } else if (try_split(c, i, mk)) {
                for (auto& x : mk) kernels.push_back(x);
            } else if (std::set<int> top; cut_for_split(c, i, &top)) {
                for (int t : top) need[t] = 1;
                again = true;
            } else if (try_row(c, i, k)) {
                kernels.push_back(k);
            } else if (try_reduce_cells(c, i, k)) {
                kernels.push_back(k);
            } else {
                std::set<int> top;
                reach_reduces(c, i, top, true);
                if (top.empty()) fail(RV_E_INVALID, fmt("internal: node %d cannot be scheduled", i));
                for (int t : top) need[t] = 1;
                again = true;
            }
        }
        if (!again) {
            p.kernels = kernels;
            // outputs that are graph inputs: plain copies
            for (size_t k = 0; k < g.outputs.size(); ++k) {
                int o = g.outputs[k];
                if (g.nodes[o].op != RV_BUFFER) continue;
                Kernel kc;
                kc.cls = KClass::EW;
                kc.domain = g.nodes[o].shape;
                Builder b{c, kc, o, Builder::EW};
                int e = b.build(o, identity(kc.domain.size()));
                std::vector<Loc> save = c.loc[o];
                c.loc[o] = {Loc{1, (int)k}};
                add_stores(c, kc, o, e, identity(kc.domain.size()));
                c.loc[o] = save;
                p.kernels.push_back(kc);
            }
            for (size_t k = 0; k < p.kernels.size(); ++k) p.kernels[k].name = fmt("rv_k%zu", k);
            return;
        }
    }
    fail(RV_E_INVALID, "internal: scheduling did not converge");
}

}  // namespace rv
