// View algebra: limn README, "Architecture" (third rule). A View is
// (shape, strides, offset, mask); reshape, permute, expand, pad and shrink
// compose into a single View without touching data, and a padded read is a
// range check that yields zero (limn README, "Reading the schedule").
//
// Reading taken where the page is silent: the mask is one half-open range
// per dim, so a reshape composes only when every masked dim passes through
// unchanged, and dims that merge must chain (stride[d] == size[d+1] *
// stride[d+1]). Anything else is RV_E_UNSUPPORTED_LAYOUT and the caller makes
// the value contiguous first.
#include <algorithm>

#include "common.hpp"

namespace rv {

static int64_t mul_checked(int64_t a, int64_t b) {
    int64_t r;
    if (__builtin_mul_overflow(a, b, &r)) fail(RV_E_INVALID, "view arithmetic overflows int64");
    return r;
}

static int64_t add_checked(int64_t a, int64_t b) {
    int64_t r;
    if (__builtin_add_overflow(a, b, &r)) fail(RV_E_INVALID, "view arithmetic overflows int64");
    return r;
}

Shape view_shape(const rv_view& v) { return Shape(v.shape, v.shape + v.ndim); }

void view_check(const rv_view& v) {
    if (v.ndim < 0 || v.ndim > RV_MAX_DIMS) fail(RV_E_INVALID, fmt("view rank %d outside [0, 8]", v.ndim));
    for (int d = 0; d < v.ndim; ++d) {
        if (v.shape[d] < 0) fail(RV_E_INVALID, fmt("view dim %d has negative size", d));
        if (v.strides[d] < 0)
            fail(RV_E_UNSUPPORTED_LAYOUT, fmt("view dim %d has a negative stride: a step other than 1 has no View", d));
        if (v.mask_lo[d] < 0 || v.mask_lo[d] > v.mask_hi[d] || v.mask_hi[d] > v.shape[d])
            fail(RV_E_INVALID, fmt("view dim %d mask [%lld, %lld) outside [0, %lld]", d, (long long)v.mask_lo[d],
                                   (long long)v.mask_hi[d], (long long)v.shape[d]));
    }
}

bool view_empty_mask(const rv_view& v) {
    for (int d = 0; d < v.ndim; ++d)
        if (v.mask_lo[d] >= v.mask_hi[d]) return true;
    return false;
}

bool view_is_contiguous(const rv_view& v) {
    if (v.offset != 0) return false;
    bool empty = false;
    for (int d = 0; d < v.ndim; ++d) empty = empty || v.shape[d] == 0;
    if (empty) {  // no element is addressed: the strides do not matter
        for (int d = 0; d < v.ndim; ++d)
            if (v.mask_lo[d] != 0 || v.mask_hi[d] != v.shape[d]) return false;
        return true;
    }
    int64_t s = 1;
    for (int d = v.ndim - 1; d >= 0; --d) {
        if (v.mask_lo[d] != 0 || v.mask_hi[d] != v.shape[d]) return false;
        if (v.shape[d] != 1 && v.strides[d] != s) return false;
        s *= v.shape[d];
    }
    return true;
}

bool view_addr_range(const rv_view& v, int64_t* lo, int64_t* hi) {
    if (view_empty_mask(v)) return false;
    int64_t a = v.offset, b = v.offset;
    for (int d = 0; d < v.ndim; ++d) {
        a = add_checked(a, mul_checked(v.mask_lo[d], v.strides[d]));
        b = add_checked(b, mul_checked(v.mask_hi[d] - 1, v.strides[d]));
    }
    *lo = a;
    *hi = b;
    return true;
}

// The outer View addresses cells of inner's shape by their row-major index.
// Starting from the lowest unmasked outer cell (index base, inner cell j0),
// each outer dim with more than one unmasked step must move exactly one inner
// dim by a whole multiple of that dim's pitch, and the inner dim must not
// carry over its size anywhere in the unmasked range; then every inner index
// is affine in the outer one and the composition is one View. An inner mask
// becomes a range on the one outer dim that moves that inner dim (or, with
// none moving it, either no constraint or an empty View).
bool view_compose(const rv_view& inner, const rv_view& outer, rv_view* out) {
    view_check(inner);
    view_check(outer);
    const int ni = inner.ndim, no = outer.ndim;
    rv_view r = outer;
    if (view_empty_mask(outer)) {  // nothing is read: any source address will do
        for (int d = 0; d < no; ++d) r.strides[d] = 0;
        r.offset = inner.offset;
        *out = r;
        return true;
    }
    int64_t pitch[RV_MAX_DIMS], total = 1;
    for (int e = ni - 1; e >= 0; --e) {
        pitch[e] = total;
        total = mul_checked(total, inner.shape[e]);
    }
    int64_t base = outer.offset;
    for (int d = 0; d < no; ++d) base = add_checked(base, mul_checked(outer.mask_lo[d], outer.strides[d]));
    if (base < 0 || base >= total) return false;
    int64_t j0[RV_MAX_DIMS], rem = base;
    for (int e = 0; e < ni; ++e) {
        j0[e] = rem / pitch[e];
        rem %= pitch[e];
    }
    int map[RV_MAX_DIMS];
    int64_t coef[RV_MAX_DIMS], span[RV_MAX_DIMS];
    int movers[RV_MAX_DIMS];
    for (int e = 0; e < ni; ++e) span[e] = j0[e], movers[e] = 0;
    for (int d = 0; d < no; ++d) {
        map[d] = -1;
        coef[d] = 0;
        const int64_t steps = outer.mask_hi[d] - outer.mask_lo[d];
        if (steps <= 1 || outer.strides[d] == 0) continue;
        int e = -1;
        for (int x = ni - 1; x >= 0; --x)
            if (inner.shape[x] > 1 && outer.strides[d] % pitch[x] == 0 && outer.strides[d] / pitch[x] < inner.shape[x]) {
                e = x;
                break;
            }
        if (e < 0) return false;
        map[d] = e;
        coef[d] = outer.strides[d] / pitch[e];
        span[e] = add_checked(span[e], mul_checked(coef[d], steps - 1));
        ++movers[e];
    }
    for (int e = 0; e < ni; ++e)
        if (span[e] >= inner.shape[e]) return false;  // a carry: not affine
    int64_t off = inner.offset;
    for (int e = 0; e < ni; ++e) off = add_checked(off, mul_checked(j0[e], inner.strides[e]));
    for (int d = 0; d < no; ++d) {
        r.strides[d] = map[d] < 0 ? 0 : mul_checked(coef[d], inner.strides[map[d]]);
        off = add_checked(off, -mul_checked(outer.mask_lo[d], r.strides[d]));
    }
    r.offset = off;
    bool empty = false;
    for (int e = 0; e < ni; ++e) {
        const int64_t lo = inner.mask_lo[e], hi = inner.mask_hi[e];
        if (lo == 0 && hi == inner.shape[e]) continue;
        if (movers[e] == 0) {
            if (j0[e] < lo || j0[e] >= hi) empty = true;
            continue;
        }
        if (movers[e] > 1) return false;
        int d = 0;
        while (map[d] != e) ++d;
        // lo <= j0 + c (i - mlo) < hi  <=>  i in [mlo + ceil((lo - j0) / c), mlo + ceil((hi - j0) / c))
        const int64_t c = coef[d], m0 = outer.mask_lo[d];
        auto ceil_div = [](int64_t a, int64_t b) { return a >= 0 ? (a + b - 1) / b : -((-a) / b); };
        const int64_t a = m0 + ceil_div(lo - j0[e], c), b = m0 + ceil_div(hi - j0[e], c);
        r.mask_lo[d] = std::max(r.mask_lo[d], std::min(a, r.shape[d]));
        r.mask_hi[d] = std::min(r.mask_hi[d], std::max(b, (int64_t)0));
        if (r.mask_hi[d] < r.mask_lo[d]) r.mask_hi[d] = r.mask_lo[d];
    }
    if (empty) {
        if (no == 0) return false;
        r.mask_lo[0] = r.mask_hi[0] = 0;
    }
    *out = r;
    return true;
}

rv_view view_contiguous(const Shape& shape, int64_t offset) {
    if (shape.size() > RV_MAX_DIMS) fail(RV_E_INVALID, fmt("rank %zu > 8", shape.size()));
    rv_view v{};
    v.ndim = (int32_t)shape.size();
    int64_t s = 1;
    for (int d = v.ndim - 1; d >= 0; --d) {
        if (shape[d] < 0) fail(RV_E_INVALID, "negative size");
        v.shape[d] = shape[d];
        v.strides[d] = shape[d] == 1 ? 0 : s;
        v.mask_lo[d] = 0;
        v.mask_hi[d] = shape[d];
        s = mul_checked(s, std::max<int64_t>(shape[d], 1));
    }
    v.offset = offset;
    return v;
}

rv_view view_permute(const rv_view& in, const std::vector<int>& perm) {
    view_check(in);
    if ((int)perm.size() != in.ndim) fail(RV_E_INVALID, "permute: rank mismatch");
    std::vector<int> seen(in.ndim, 0);
    for (int p : perm) {
        if (p < 0 || p >= in.ndim || seen[p]++) fail(RV_E_INVALID, "permute: not a permutation");
    }
    rv_view o = in;
    for (int d = 0; d < in.ndim; ++d) {
        o.shape[d] = in.shape[perm[d]];
        o.strides[d] = in.strides[perm[d]];
        o.mask_lo[d] = in.mask_lo[perm[d]];
        o.mask_hi[d] = in.mask_hi[perm[d]];
    }
    return o;
}

rv_view view_expand(const rv_view& in, const Shape& shape) {
    view_check(in);
    if ((int)shape.size() != in.ndim) fail(RV_E_INVALID, "expand: rank mismatch");
    rv_view o = in;
    for (int d = 0; d < in.ndim; ++d) {
        if (shape[d] == in.shape[d]) continue;
        if (in.shape[d] != 1 || shape[d] < 0)
            fail(RV_E_INVALID, fmt("expand: dim %d of size %lld cannot become %lld", d, (long long)in.shape[d],
                                   (long long)shape[d]));
        bool inside = in.mask_lo[d] == 0 && in.mask_hi[d] == 1;
        o.shape[d] = shape[d];
        o.strides[d] = 0;
        o.mask_lo[d] = 0;
        o.mask_hi[d] = inside ? shape[d] : 0;
    }
    return o;
}

rv_view view_pad(const rv_view& in, const Shape& before, const Shape& after) {
    view_check(in);
    if ((int)before.size() != in.ndim || (int)after.size() != in.ndim) fail(RV_E_INVALID, "pad: rank mismatch");
    rv_view o = in;
    for (int d = 0; d < in.ndim; ++d) {
        if (before[d] < 0 || after[d] < 0) fail(RV_E_INVALID, "pad: negative width");
        o.shape[d] = add_checked(add_checked(in.shape[d], before[d]), after[d]);
        o.offset = add_checked(o.offset, -mul_checked(before[d], in.strides[d]));
        o.mask_lo[d] = in.mask_lo[d] + before[d];
        o.mask_hi[d] = in.mask_hi[d] + before[d];
    }
    return o;
}

rv_view view_shrink(const rv_view& in, const Shape& lo, const Shape& hi) {
    view_check(in);
    if ((int)lo.size() != in.ndim || (int)hi.size() != in.ndim) fail(RV_E_INVALID, "shrink: rank mismatch");
    rv_view o = in;
    for (int d = 0; d < in.ndim; ++d) {
        if (!(0 <= lo[d] && lo[d] <= hi[d] && hi[d] <= in.shape[d]))
            fail(RV_E_INVALID, fmt("shrink: [%lld, %lld) outside dim %d of size %lld", (long long)lo[d],
                                   (long long)hi[d], d, (long long)in.shape[d]));
        o.shape[d] = hi[d] - lo[d];
        o.offset = add_checked(o.offset, mul_checked(lo[d], in.strides[d]));
        int64_t ml = std::max<int64_t>(in.mask_lo[d] - lo[d], 0);
        int64_t mh = std::min<int64_t>(in.mask_hi[d] - lo[d], o.shape[d]);
        if (mh < ml) ml = mh = 0;
        o.mask_lo[d] = ml;
        o.mask_hi[d] = mh;
    }
    return o;
}

rv_view view_reshape(const rv_view& in, const Shape& shape) {
    view_check(in);
    if (shape.size() > RV_MAX_DIMS) fail(RV_E_INVALID, "reshape: rank > 8");
    for (int64_t s : shape)
        if (s < 0) fail(RV_E_INVALID, "reshape: negative size");
    const Shape old = view_shape(in);
    if (numel(old) != numel(shape))
        fail(RV_E_INVALID, "reshape: " + shape_str(old) + " and " + shape_str(shape) + " differ in size");
    if (numel(shape) == 0) return view_contiguous(shape, in.offset);
    if (view_empty_mask(in)) {
        if (shape.empty()) fail(RV_E_UNSUPPORTED_LAYOUT, "reshape: a fully masked view has no rank-0 form");
        rv_view o = view_contiguous(shape, 0);
        o.mask_lo[0] = o.mask_hi[0] = 0;
        return o;
    }
    if (view_is_contiguous(in)) return view_contiguous(shape, in.offset);

    struct Dim {
        int64_t size, stride, lo, hi;
    };
    std::vector<Dim> a;  // non-size-1 dims of the input
    for (int d = 0; d < in.ndim; ++d)
        if (in.shape[d] != 1) a.push_back({in.shape[d], in.strides[d], in.mask_lo[d], in.mask_hi[d]});
    std::vector<int> b;  // positions of non-size-1 dims of the output
    for (int d = 0; d < (int)shape.size(); ++d)
        if (shape[d] != 1) b.push_back(d);

    rv_view o{};
    o.ndim = (int32_t)shape.size();
    o.offset = in.offset;
    for (int d = 0; d < o.ndim; ++d) {
        o.shape[d] = shape[d];
        o.strides[d] = 0;
        o.mask_lo[d] = 0;
        o.mask_hi[d] = shape[d];
    }
    size_t i = 0, j = 0;
    while (i < a.size() && j < b.size()) {
        size_t i0 = i, j0 = j;
        int64_t pi = a[i].size, pj = shape[b[j]];
        while (pi != pj) {
            if (pi < pj) {
                if (++i >= a.size()) fail(RV_E_INVALID, "reshape: size bookkeeping");
                pi *= a[i].size;
            } else {
                if (++j >= b.size()) fail(RV_E_INVALID, "reshape: size bookkeeping");
                pj *= shape[b[j]];
            }
        }
        if (i == i0 && j == j0) {
            o.strides[b[j]] = a[i].stride;
            o.mask_lo[b[j]] = a[i].lo;
            o.mask_hi[b[j]] = a[i].hi;
        } else {
            for (size_t k = i0; k <= i; ++k) {
                if (a[k].lo != 0 || a[k].hi != a[k].size)
                    fail(RV_E_UNSUPPORTED_LAYOUT, "reshape: a masked dim would be split or merged; make the value "
                                                  "contiguous first");
                if (k < i && a[k].stride != a[k + 1].size * a[k + 1].stride)
                    fail(RV_E_UNSUPPORTED_LAYOUT, "reshape: dims whose strides do not chain cannot merge into one "
                                                  "View; make the value contiguous first");
            }
            int64_t s = a[i].stride;
            for (size_t k = j + 1; k-- > j0;) {
                o.strides[b[k]] = s;
                s = mul_checked(s, shape[b[k]]);
            }
        }
        ++i;
        ++j;
    }
    return o;
}

}  // namespace rv
