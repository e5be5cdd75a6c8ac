// Shared host-side definitions of the library (not part of the C ABI).
#pragma once

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "rv.h"

namespace rv {

using Shape = std::vector<int64_t>;

// Every internal failure is thrown as an Error and turned into a status at
// the C boundary (no exception crosses the ABI).
struct Error {
    rv_status status;
    std::string msg;
};

[[noreturn]] inline void fail(rv_status s, const std::string& msg) { throw Error{s, msg}; }

inline std::string fmt(const char* f, ...) {
    char buf[1024];
    va_list ap;
    va_start(ap, f);
    vsnprintf(buf, sizeof buf, f, ap);
    va_end(ap);
    return buf;
}

inline bool dtype_valid(int dt) { return dt >= RV_F32 && dt <= RV_I8; }
inline bool is_float(int dt) { return dt == RV_F32 || dt == RV_BF16 || dt == RV_F16 || dt == RV_F64; }
inline bool is_int(int dt) { return dt == RV_I32 || dt == RV_I16 || dt == RV_I8; }
inline bool is_half(int dt) { return dt == RV_BF16 || dt == RV_F16; }

inline int dtype_size(int dt) {
    switch (dt) {
        case RV_F32: case RV_I32: return 4;
        case RV_F64: return 8;
        case RV_BF16: case RV_F16: case RV_I16: return 2;
        case RV_I8: return 1;
    }
    return 0;
}

inline const char* dtype_name(int dt) {
    static const char* n[] = {"f32", "bf16", "f16", "f64", "i32", "i16", "i8"};
    return dtype_valid(dt) ? n[dt] : "?";
}

inline const char* op_name(int op) {
    static const char* n[] = {"BUFFER", "CONST", "VIEW", "NEG", "EXP", "LOG", "SQRT", "RECIP",
                              "CAST", "ADD", "MUL", "CMPLT", "WHERE", "SUM", "MAX", "CONTIGUOUS",
                              "GATHER", "SCATTER", "ASSIGN", "CUSTOM"};
    return (op >= 0 && op <= RV_CUSTOM) ? n[op] : "?";
}

inline int64_t numel(const Shape& s) {
    int64_t n = 1;
    for (int64_t d : s) n *= d;
    return n;
}

// A tuning knob from the environment (unset or empty: the default).
inline int env_int(const char* name, int def) {
    const char* s = getenv(name);
    return (s && *s) ? atoi(s) : def;
}

inline std::string shape_str(const Shape& s) {
    std::string r = "(";
    for (size_t i = 0; i < s.size(); ++i) r += (i ? "," : "") + std::to_string(s[i]);
    return r + ")";
}

// ---- views (view.cpp) ----
rv_view view_contiguous(const Shape& shape, int64_t offset = 0);
rv_view view_reshape(const rv_view& in, const Shape& shape);
rv_view view_permute(const rv_view& in, const std::vector<int>& perm);
rv_view view_expand(const rv_view& in, const Shape& shape);
rv_view view_pad(const rv_view& in, const Shape& before, const Shape& after);
rv_view view_shrink(const rv_view& in, const Shape& lo, const Shape& hi);
void view_check(const rv_view& v);                      // well-formed: ndim, shape, mask, strides
bool view_empty_mask(const rv_view& v);                 // no cell is in the mask
bool view_is_contiguous(const rv_view& v);              // row-major, offset 0, unmasked
// Closed-form range of the addresses an in-mask cell can form: [lo, hi].
// Returns false when no cell is in the mask.
bool view_addr_range(const rv_view& v, int64_t* lo, int64_t* hi);
Shape view_shape(const rv_view& v);
// A View `outer` over the row-major cells of the View `inner`, as one View
// of inner's source; false when no single View expresses it (a carry across
// an inner dim, or one inner mask reached by several outer dims)
bool view_compose(const rv_view& inner, const rv_view& outer, rv_view* out);

}  // namespace rv
