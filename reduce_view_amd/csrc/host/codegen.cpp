// Code generation: renders every lowered kernel as HIP source for gfx950.
// Shapes, strides, offsets and masks are baked in as constants, so each View
// becomes plain integer arithmetic and range checks (limn README, "Reading
// the schedule": views lower to index arithmetic; the printed nest is exactly
// what the compiled backends run).
//
// Numerics follow the pages' primitives one for one: every value has the
// dtype of its graph node; float16/bfloat16 values are computed in float32
// and rounded once per node; ints wrap; the source is compiled with
// -ffp-contract=off so a MUL and the ADD after it stay two roundings.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <functional>
#include <set>
#include <sstream>

#include "graph.hpp"

namespace rv {

extern const char* const kDeviceHeader;

namespace {

std::string st(int dt) {  // storage type
    switch (dt) {
        case RV_F32: return "float";
        case RV_BF16: return "unsigned short";
        case RV_F16: return "_Float16";
        case RV_F64: return "double";
        case RV_I32: return "int";
        case RV_I16: return "short";
        case RV_I8: return "signed char";
    }
    return "?";
}

std::string vt(int dt) {  // register type
    if (dt == RV_F64) return "double";
    if (is_int(dt)) return "int";
    return "float";
}

std::string ld(int dt, const std::string& e) {  // storage -> register
    if (dt == RV_BF16) return "rv_bf2f(" + e + ")";
    if (dt == RV_F16) return "((float)(" + e + "))";
    if (is_int(dt)) return "((int)(" + e + "))";
    return e;
}

std::string sv(int dt, const std::string& e) {  // register -> storage
    switch (dt) {
        case RV_BF16: return "rv_f2bf(" + e + ")";
        case RV_F16: return "((_Float16)(" + e + "))";
        case RV_I16: return "((short)(" + e + "))";
        case RV_I8: return "((signed char)(" + e + "))";
    }
    return e;
}

std::string round_to(int dt, const std::string& e) {  // float32 result -> node dtype
    if (dt == RV_BF16) return "rv_rbf(" + e + ")";
    if (dt == RV_F16) return "rv_rhf(" + e + ")";
    return e;
}

std::string wrap_int(int dt, const std::string& e) {
    if (dt == RV_I16) return "((int)(short)(" + e + "))";
    if (dt == RV_I8) return "((int)(signed char)(" + e + "))";
    return "((int)(" + e + "))";
}

std::string flit(double v) {  // exact float32 literal
    float f = (float)v;
    if (std::isnan(f)) return "__builtin_nanf(\"\")";
    if (std::isinf(f)) return f > 0 ? "__builtin_inff()" : "(-__builtin_inff())";
    char b[64];
    snprintf(b, sizeof b, "%af", (double)f);
    return b;
}

std::string dlit(double v) {
    if (std::isnan(v)) return "__builtin_nan(\"\")";
    if (std::isinf(v)) return v > 0 ? "__builtin_inf()" : "(-__builtin_inf())";
    char b[64];
    snprintf(b, sizeof b, "%a", v);
    return b;
}

float round_bf16_host(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return f;
    u += 0x7fffu + ((u >> 16) & 1u);
    u &= 0xffff0000u;
    memcpy(&f, &u, 4);
    return f;
}

std::string const_lit(int dt, double v) {
    switch (dt) {
        case RV_F32: return flit(v);
        case RV_BF16: return flit(round_bf16_host((float)v));
        case RV_F16: return flit((float)(_Float16)(float)v);
        case RV_F64: return dlit(v);
        case RV_I32: return fmt("((int)%lld)", (long long)(int32_t)(int64_t)v);
        case RV_I16: return fmt("((int)%d)", (int)(int16_t)(int64_t)v);
        case RV_I8: return fmt("((int)%d)", (int)(int8_t)(int64_t)v);
    }
    return "0";
}

std::string zero_of(int dt) { return dt == RV_F64 ? "0.0" : (is_int(dt) ? "0" : "0.0f"); }

// Value of one elementwise op from operand expressions.
std::string op_code(const Kernel& k, const Ex& e, const std::string& A, const std::string& B, const std::string& C) {
    const int dt = e.dtype;
    const bool fl = is_float(dt);
    switch (e.op) {
        case RV_NEG:
            if (fl) return "(-(" + A + "))";
            return dt == RV_I32 ? "((int)(0u - (unsigned)(" + A + ")))" : wrap_int(dt, "-(" + A + ")");
        case RV_EXP: return dt == RV_F64 ? "exp(" + A + ")" : round_to(dt, "expf(" + A + ")");
        case RV_LOG: return dt == RV_F64 ? "log(" + A + ")" : round_to(dt, "logf(" + A + ")");
        case RV_SQRT: return dt == RV_F64 ? "sqrt(" + A + ")" : round_to(dt, "sqrtf(" + A + ")");
        case RV_RECIP: return dt == RV_F64 ? "(1.0 / (" + A + "))" : round_to(dt, "(1.0f / (" + A + "))");
        case RV_ADD:
        case RV_MUL: {
            const char* o = e.op == RV_ADD ? " + " : " * ";
            if (fl) return round_to(dt, "((" + A + ")" + o + "(" + B + "))");
            if (dt == RV_I32) return "((int)((unsigned)(" + A + ")" + o + "(unsigned)(" + B + ")))";
            return wrap_int(dt, "(" + A + ")" + o + "(" + B + ")");
        }
        case RV_CMPLT: return "(((" + A + ") < (" + B + ")) ? 1 : 0)";
        case RV_WHERE: return "(((" + A + ") != 0) ? (" + B + ") : (" + C + "))";
        case RV_CAST: {
            const int s = k.ex[e.a].dtype;
            if (s == dt) return A;
            if (is_int(dt)) {
                if (is_int(s)) return wrap_int(dt, A);
                return wrap_int(dt, "(int)(" + A + ")");
            }
            if (dt == RV_F64) return "((double)(" + A + "))";
            // a value headed for a half width is a float32 first (float64
            // and int sources round twice, as the oracle and torch do)
            if (s == RV_F64) return round_to(dt, "((float)(" + A + "))");
            if (is_int(s)) return round_to(dt, "((float)(" + A + "))");
            return round_to(dt, A);
        }
    }
    fail(RV_E_INVALID, fmt("internal: no code for op %d", e.op));
}

// Accumulator of a SUM / MAX in a row kernel: float for float32 and the
// half widths (widened), double for float64, and for ints an unsigned total
// (a SUM wraps modulo 2^32, exactly as the serial fold does) or an int (MAX).
struct RedType {
    std::string t, ident, fin;
    bool sum = true, isint = false, isdbl = false;
    RedType(int op, int dt) {
        sum = op == RV_SUM;
        isint = is_int(dt);
        isdbl = dt == RV_F64;
        if (isdbl) {
            t = "double";
            ident = sum ? "0.0" : "(-__builtin_inf())";
        } else if (isint) {
            t = sum ? "unsigned" : "int";
            ident = sum ? "0u" : (dt == RV_I32 ? "(-2147483647 - 1)" : (dt == RV_I16 ? "(-32768)" : "(-128)"));
        } else {
            t = "float";
            ident = sum ? "0.0f" : "(-__builtin_inff())";
        }
    }
    // acc (op) v for a value v of the register type
    std::string fold(const std::string& acc, const std::string& v) const {
        if (sum) return acc + " + " + (isint ? "(unsigned)(" + v + ")" : "(" + v + ")");
        if (isdbl) return "rv_maxd(" + acc + ", " + v + ")";
        if (isint) return "((" + v + ") > " + acc + " ? (" + v + ") : " + acc + ")";
        return "rv_maxf(" + acc + ", " + v + ")";
    }
    std::string result(int dt, const std::string& acc) const { return isint ? wrap_int(dt, acc) : round_to(dt, acc); }
};

struct Gen {
    const Program& p;
    const Kernel& k;
    std::ostringstream o;
    std::vector<Loc> params;
    std::vector<char> written;
    std::vector<int> param_dtype;
    std::vector<char> live;
    std::string I;  // index type
    int rank = 0;

    Gen(const Program& p_, const Kernel& k_) : p(p_), k(k_) {
        rank = (int)k.domain.size();
        live.assign(k.ex.size(), 0);
        std::function<void(int)> mark = [&](int e) {
            if (e < 0 || live[e]) return;
            live[e] = 1;
            mark(k.ex[e].a);
            mark(k.ex[e].b);
            mark(k.ex[e].c);
        };
        for (auto& s : k.stores) mark(s.ex);
        if (k.cls == KClass::SPLIT)  // its one reduce feeds the partials, not a store
            for (size_t e = 0; e < k.ex.size(); ++e)
                if (k.ex[e].op == RV_SUM || k.ex[e].op == RV_MAX) mark((int)e);
        int64_t mx = numel(k.domain);
        auto upd = [&](const rv_view& v) {
            int64_t lo, hi;
            if (view_addr_range(v, &lo, &hi)) mx = std::max({mx, hi + 1, -lo + 1});
        };
        for (auto& L : k.leaves)
            if (!L.zero) upd(L.v);
        for (auto& s : k.stores) upd(s.v);
        for (auto& e : k.ex) {  // a gathered read reaches index * g_stride further
            int64_t lo, hi;
            if (e.op != RV_GATHER || k.leaves[e.leaf].zero || !view_addr_range(k.leaves[e.leaf].v, &lo, &hi)) continue;
            const int64_t far = (e.g_hi - e.g_lo) * std::abs(e.g_stride);
            mx = std::max({mx, hi + far + 1, -(lo - far) + 1});
        }
        if (k.cls == KClass::SCATTER) mx = std::max(mx, numel(k.sc_out_shape) + 1);
        I = mx < (int64_t(1) << 30) ? "int" : "long long";
        const char* nt = getenv("RV_NT");
        nt_on = !(nt && std::string(nt) == "0");
    }

    int param_of(const Loc& L, int dtype, bool write) {
        for (size_t i = 0; i < params.size(); ++i)
            if (params[i] == L) {
                written[i] = written[i] || write;
                return (int)i;
            }
        params.push_back(L);
        written.push_back(write);
        param_dtype.push_back(dtype);
        return (int)params.size() - 1;
    }

    std::string pname(const Loc& L, int dtype, bool write) { return fmt("p%d", param_of(L, dtype, write)); }

    std::string lit(int64_t v) { return I == "int" ? std::to_string(v) : std::to_string(v) + "LL"; }

    // address of leaf/store view at domain index expressions idx[d]
    std::string addr(const rv_view& v, const std::vector<std::string>& idx) {
        std::string s = lit(v.offset);
        for (int d = 0; d < rank; ++d) {
            if (v.strides[d] == 0 || idx[d].empty()) continue;
            s += " + (" + idx[d] + ")" + (v.strides[d] == 1 ? "" : " * " + lit(v.strides[d]));
        }
        return s;
    }

    bool masked(const rv_view& v, int d) const { return !(v.mask_lo[d] == 0 && v.mask_hi[d] == k.domain[d]); }

    // mask condition for dims in `dims` (empty string: always true)
    std::string mask_cond(const rv_view& v, const std::vector<std::string>& idx, const std::vector<int>& dims) {
        std::string s;
        for (int d : dims) {
            if (!masked(v, d)) continue;
            if (!s.empty()) s += " && ";
            s += fmt("(%s) >= %s && (%s) < %s", idx[d].c_str(), lit(v.mask_lo[d]).c_str(), idx[d].c_str(),
                     lit(v.mask_hi[d]).c_str());
        }
        return s;
    }

    std::string signature() {
        std::string s;
        for (size_t i = 0; i < params.size(); ++i) {
            s += i ? ", " : "";
            s += (written[i] ? "" : "const ") + st(param_dtype[i]) + "* __restrict__ " + fmt("p%zu", i);
        }
        return s;
    }

    std::string header() {
        // a 256 x 256 contraction tile on 4 waves keeps 256 accumulators per
        // lane: one wave per SIMD, so the whole register file is the wave's.
        // The attention forward (4 waves, one per SIMD) asks for several
        // waves per SIMD: 4 at head width 32, 3 at 64, 2 at 128, which also
        // keeps its matrix results in ordinary vector registers (with a
        // budget of more than 256 registers the compiler places them in the
        // accumulation registers and moves every score in and out)
        std::string occ;
        if (k.cls == KClass::MFMA && !k.mfma_slices) occ = "__attribute__((amdgpu_waves_per_eu(1, 1))) ";
        if (k.cls == KClass::ATTN && !k.attn_merge) {
            const int64_t D = k.domain[2];
            occ = fmt("__attribute__((amdgpu_waves_per_eu(%d))) ", D == 32 ? 4 : D == 64 ? 3 : 2);
        }
        return "extern \"C\" __global__ void __launch_bounds__(" + std::to_string(k.block[0]) + ") " + occ + k.name +
               "(" + signature() + ")";
    }

    // a load is streaming (nontemporal) when no domain dim of size > 1 has
    // stride 0, i.e. every cell is read once; stores always stream
    bool streaming(const Leaf& L) const {
        if (!nt_on) return false;
        for (int d = 0; d < rank; ++d)
            if (k.domain[d] > 1 && L.v.strides[d] == 0) return false;
        return true;
    }
    std::string vload(const Leaf& L, int n, const std::string& ptr) const {
        bool nt = streaming(L) && dtype_size(L.dtype) * n >= 4;
        return std::string(nt ? "rv_ldv_nt<" : "rv_ldv<") + st(L.dtype) + ", " + std::to_string(n) + ">(" + ptr + ")";
    }
    std::string vstore(int dtype, int n, const std::string& ptr, const std::string& val) const {
        bool nt = nt_on && dtype_size(dtype) * n >= 4;
        return std::string(nt ? "rv_stv_nt<" : "rv_stv<") + st(dtype) + ", " + std::to_string(n) + ">(" + ptr + ", " + val +
               ")";
    }
    bool nt_on = true;

    bool leaf_vec_ok(const Leaf& L, int along, int vw) {
        if (vw <= 1 || L.v.strides[along] != 1) return false;
        if (L.v.offset % vw) return false;
        for (int d = 0; d < rank; ++d)
            if (d != along && k.domain[d] > 1 && L.v.strides[d] % vw) return false;
        return true;
    }

    // Scalar code for value `e` (its operands first, each once) at domain
    // index expressions idx; the value is named s<e><sfx>.
    void scalar(std::ostringstream& b, int e, const std::vector<std::string>& idx, const std::string& ind,
                const std::string& sfx, std::vector<char>& done) {
        if (e < 0 || done[e]) return;
        const Ex& x = k.ex[e];
        scalar(b, x.a, idx, ind, sfx, done);
        scalar(b, x.b, idx, ind, sfx, done);
        scalar(b, x.c, idx, ind, sfx, done);
        done[e] = 1;
        const std::string V = fmt("s%d%s", e, sfx.c_str());
        auto E = [&](int i) { return i < 0 ? std::string() : fmt("s%d%s", i, sfx.c_str()); };
        std::vector<int> all;
        for (int d = 0; d < rank; ++d) all.push_back(d);
        b << ind << "const " << vt(x.dtype) << " " << V << " = ";
        if (x.op == RV_BUFFER || x.op == RV_GATHER) {
            const Leaf& L = k.leaves[x.leaf];
            if (L.zero || (x.op == RV_GATHER && x.g_hi <= x.g_lo)) {
                b << zero_of(x.dtype) << ";\n";
                return;
            }
            std::string mc = mask_cond(L.v, idx, all);
            std::string a = addr(L.v, idx);
            if (x.op == RV_GATHER) {
                const std::string T = E(x.a);
                mc = fmt("(%s) >= %lld && (%s) < %lld", T.c_str(), (long long)x.g_lo, T.c_str(), (long long)x.g_hi) +
                     (mc.empty() ? "" : " && " + mc);
                a += " + (" + I + ")((" + T + ") - " + std::to_string(x.g_lo) + ") * " + lit(x.g_stride);
            }
            const std::string P = pname(L.loc, L.dtype, false);
            b << (mc.empty() ? "" : "(" + mc + ") ? ") << ld(L.dtype, P + "[" + a + "]")
              << (mc.empty() ? "" : " : " + zero_of(x.dtype)) << ";\n";
        } else if (x.op == RV_CONST) {
            b << const_lit(x.dtype, x.cval) << ";\n";
        } else {
            b << op_code(k, x, E(x.a), E(x.b), E(x.c)) << ";\n";
        }
    }

    void gather_rowmajor(std::ostringstream& b, const Ex& x, int u, const std::string& V, int VW, int64_t NX,
                         bool full_chunks, const std::vector<int>& outer, const std::vector<std::string>& idx);
    std::string gen();
    std::string gen_scatter();
    std::string gen_rowmajor();
    std::string gen_tiled();
    std::string gen_row();
    std::string gen_row_stream();
    std::string gen_attn();
    std::string gen_cells();
    std::string gen_split_cols();
    std::string gen_fold_cells();
    std::string gen_fold();
    std::string gen_gemm();
};

// ---------------------------------------------------------------------------
// EW, row-major plan: every thread takes chunks of VW consecutive cells of
// the innermost dim; operands that are contiguous along it are read as one
// vector, stride-0 operands once, others cell by cell.
// ---------------------------------------------------------------------------
// GATHER in the row-major plan: cell by cell, the data read at its View's
// address plus index * g_stride; when the index is the same across the
// chunk (constant along the lane dim) and the data is contiguous along it,
// one vector read.
void Gen::gather_rowmajor(std::ostringstream& b, const Ex& x, int u, const std::string& V, int VW, int64_t NX,
                          bool full_chunks, const std::vector<int>& outer, const std::vector<std::string>& idx) {
    const int X = rank - 1;
    const Leaf& L = k.leaves[x.leaf];
    if (L.zero || x.g_hi <= x.g_lo) return;  // every cell reads zero
    const std::string P = pname(L.loc, L.dtype, false);
    const std::string xs = "x" + std::to_string(u);
    const std::string T = fmt("e%d_%d", x.a, u);
    std::string rowok = "cv" + std::to_string(u);
    const std::string oc = mask_cond(L.v, idx, outer);
    if (!oc.empty()) rowok += " && " + oc;
    auto idx0 = idx;
    idx0[X] = "";
    const std::string base = addr(L.v, idx0);
    const std::string inr = fmt("%s >= %lld && %s < %lld", "t", (long long)x.g_lo, "t", (long long)x.g_hi);
    b << "    {\n";
    const int64_t gs = x.g_stride;
    if (VW > 1 && ex_invariant(k, x.a, X) && leaf_vec_ok(L, X, VW) && gs % VW == 0) {
        std::string xm = masked(L.v, X) ? fmt(" && %s >= %s && %s + %d <= %s", xs.c_str(), lit(L.v.mask_lo[X]).c_str(),
                                              xs.c_str(), VW, lit(L.v.mask_hi[X]).c_str())
                                        : "";
        std::string fullc = full_chunks ? "" : fmt(" && %s + %d <= %s", xs.c_str(), VW, lit(NX).c_str());
        b << "      const int t = " << T << "[0];\n";
        b << "      if (" << rowok << " && " << inr << xm << fullc << ") {\n";
        b << "        const rv_pack<" << st(L.dtype) << ", " << VW << "> v = rv_ldv<" << st(L.dtype) << ", " << VW << ">("
          << P << " + " << base << " + " << xs << " + (" << I << ")(t - " << x.g_lo << ") * " << lit(gs) << ");\n";
        b << "        for (int q = 0; q < " << VW << "; ++q) " << V << "[q] = " << ld(L.dtype, "v.v[q]") << ";\n";
        b << "      } else\n";
    }
    b << "      for (int q = 0; q < " << VW << "; ++q) {\n";
    b << "        const " << I << " x = " << xs << " + q;\n";
    b << "        const int t = " << T << "[q];\n";
    auto idxq = idx;
    idxq[X] = "x";
    std::string xc = mask_cond(L.v, idxq, {X});
    b << "        if (" << rowok << " && x < " << lit(NX) << (xc.empty() ? "" : " && " + xc) << " && " << inr << ") "
      << V << "[q] = " << ld(L.dtype, P + "[" + addr(L.v, idxq) + " + (" + I + ")(t - " + std::to_string(x.g_lo) +
                             ") * " + lit(gs) + "]")
      << ";\n";
    b << "      }\n    }\n";
}

std::string Gen::gen_rowmajor() {
    const int X = rank - 1;
    int VW = 1, U = 4;  // plan values (lower.cpp)
    sscanf(k.plan_json.c_str(), "\"vec\":%d,\"unroll\":%d", &VW, &U);
    const int64_t NX = k.domain[X];
    const int64_t CPR = (NX + VW - 1) / VW;
    const int64_t TOTAL = CPR * (numel(k.domain) / NX);
    const bool full_chunks = NX % VW == 0;
    std::ostringstream b;
    b << "  const " << I << " TOTAL = " << lit(TOTAL) << ";\n";
    b << "  const " << I << " STEP = (" << I << ")gridDim.x * " << 256 * U << ";\n";
    b << "  for (" << I << " cb = (" << I << ")blockIdx.x * " << 256 * U << " + threadIdx.x; cb < TOTAL; cb += STEP) {\n";
    std::vector<int> outer;
    for (int d = 0; d < X; ++d) outer.push_back(d);
    // loads for all U chunks first, then compute and store
    for (int u = 0; u < U; ++u) {
        b << "    const " << I << " c" << u << " = cb + " << 256 * u << ";\n";
        b << "    const bool cv" << u << " = c" << u << " < TOTAL;\n";
        b << "    const " << I << " row" << u << " = c" << u << " / " << lit(CPR) << ";\n";
        b << "    const " << I << " x" << u << " = (c" << u << " - row" << u << " * " << lit(CPR) << ") * " << VW << ";\n";
        // outer indices
        std::string rem = "row" + std::to_string(u);
        for (int d = X - 1; d >= 0; --d) {
            b << "    const " << I << " i" << d << "_" << u << " = " << rem << " % " << lit(k.domain[d]) << ";\n";
            if (d > 0) {
                b << "    const " << I << " q" << d << "_" << u << " = " << rem << " / " << lit(k.domain[d]) << ";\n";
                rem = "q" + std::to_string(d) + "_" + std::to_string(u);
            }
        }
    }
    auto idx_of = [&](int u, const std::string& x) {
        std::vector<std::string> idx(rank);
        for (int d = 0; d < X; ++d) idx[d] = fmt("i%d_%d", d, u);
        idx[X] = x;
        return idx;
    };
    // leaf loads
    for (size_t li = 0; li < k.leaves.size(); ++li) {
        const Leaf& L = k.leaves[li];
        bool used = false;
        for (size_t e = 0; e < k.ex.size(); ++e)
            if (live[e] && k.ex[e].op == RV_BUFFER && k.ex[e].leaf == (int)li) used = true;
        if (!used || L.zero) continue;
        std::string P = pname(L.loc, L.dtype, false);
        for (int u = 0; u < U; ++u) {
            std::string xs = "x" + std::to_string(u);
            auto idx = idx_of(u, xs);
            std::string base_idx_cond = mask_cond(L.v, idx, outer);
            std::string rowok = "cv" + std::to_string(u) + (base_idx_cond.empty() ? "" : " && " + base_idx_cond);
            std::string V = fmt("l%zu_%d", li, u);
            b << "    " << vt(L.dtype) << " " << V << "[" << VW << "];\n";
            auto idx0 = idx;
            idx0[X] = "";
            std::string base = addr(L.v, idx0);
            if (L.v.strides[X] == 0 && !masked(L.v, X)) {
                b << "    { const " << vt(L.dtype) << " s = (" << rowok << ") ? " << ld(L.dtype, P + "[" + base + "]")
                  << " : " << zero_of(L.dtype) << ";\n";
                b << "      for (int q = 0; q < " << VW << "; ++q) " << V << "[q] = s; }\n";
                continue;
            }
            bool vec = leaf_vec_ok(L, X, VW);
            std::string xm = masked(L.v, X) ? fmt(" && %s >= %s && %s + %d <= %s", xs.c_str(), lit(L.v.mask_lo[X]).c_str(),
                                                  xs.c_str(), VW, lit(L.v.mask_hi[X]).c_str())
                                            : "";
            std::string fullc = full_chunks ? "" : fmt(" && %s + %d <= %s", xs.c_str(), VW, lit(NX).c_str());
            b << "    {\n";
            if (vec) {
                b << "      if (" << rowok << xm << fullc << ") {\n";
                b << "        const rv_pack<" << st(L.dtype) << ", " << VW << "> v = "
                  << vload(L, VW, P + " + " + base + " + " + xs) << ";\n";
                b << "        for (int q = 0; q < " << VW << "; ++q) " << V << "[q] = " << ld(L.dtype, "v.v[q]") << ";\n";
                b << "      } else\n";
            }
            b << "      for (int q = 0; q < " << VW << "; ++q) {\n";
            b << "        const " << I << " x = " << xs << " + q;\n";
            auto idxq = idx;
            idxq[X] = "x";
            std::string xc = mask_cond(L.v, idxq, {X});
            b << "        " << V << "[q] = (" << rowok << " && x < " << lit(NX) << (xc.empty() ? "" : " && " + xc)
              << ") ? " << ld(L.dtype, P + "[" + addr(L.v, idxq) + "]") << " : " << zero_of(L.dtype) << ";\n";
            b << "      }\n    }\n";
        }
    }
    // expressions
    for (int u = 0; u < U; ++u) {
        for (size_t e = 0; e < k.ex.size(); ++e) {
            if (!live[e]) continue;
            const Ex& x = k.ex[e];
            std::string V = fmt("e%zu_%d", e, u);
            b << "    " << vt(x.dtype) << " " << V << "[" << VW << "];\n";
            b << "    for (int q = 0; q < " << VW << "; ++q) " << V << "[q] = ";
            if (x.op == RV_GATHER) {
                b << zero_of(x.dtype) << ";\n";
                gather_rowmajor(b, x, u, V, VW, NX, full_chunks, outer, idx_of(u, "x" + std::to_string(u)));
                continue;
            }
            if (x.op == RV_BUFFER) {
                if (k.leaves[x.leaf].zero)
                    b << zero_of(x.dtype);
                else
                    b << fmt("l%d_%d[q]", x.leaf, u);
            } else if (x.op == RV_CONST) {
                b << const_lit(x.dtype, x.cval);
            } else {
                auto E = [&](int i) { return i < 0 ? std::string() : fmt("e%d_%d[q]", i, u); };
                b << op_code(k, x, E(x.a), E(x.b), E(x.c));
            }
            b << ";\n";
        }
        // stores
        for (const Store& s : k.stores) {
            std::string P = pname(s.loc, s.dtype, true);
            std::string xs = "x" + std::to_string(u);
            auto idx = idx_of(u, xs);
            auto idx0 = idx;
            idx0[X] = "";
            std::string base = addr(s.v, idx0);
            std::string cv = "cv" + std::to_string(u);
            std::string V = fmt("e%d_%d", s.ex, u);
            bool vec = s.v.strides[X] == 1 && VW > 1 && s.v.offset % VW == 0;
            for (int d = 0; d < X; ++d)
                if (k.domain[d] > 1 && s.v.strides[d] % VW) vec = false;
            std::string fullc = full_chunks ? "" : fmt(" && %s + %d <= %s", xs.c_str(), VW, lit(NX).c_str());
            b << "    {\n";
            if (vec) {
                b << "      if (" << cv << fullc << ") {\n        rv_pack<" << st(s.dtype) << ", " << VW << "> v;\n";
                b << "        for (int q = 0; q < " << VW << "; ++q) v.v[q] = " << sv(s.dtype, V + "[q]") << ";\n";
                b << "        " << vstore(s.dtype, VW, P + " + " + base + " + " + xs, "v") << ";\n";
                b << "      } else\n";
            }
            b << "      for (int q = 0; q < " << VW << "; ++q) {\n";
            b << "        const " << I << " x = " << xs << " + q;\n";
            auto idxq = idx;
            idxq[X] = "x";
            b << "        if (" << cv << " && x < " << lit(NX) << ") " << P << "[" << addr(s.v, idxq) << "] = "
              << sv(s.dtype, V + "[q]") << ";\n";
            b << "      }\n    }\n";
        }
    }
    b << "  }\n";
    return b.str();
}

// ---------------------------------------------------------------------------
// EW, tiled plan (transpose, and chains with a permuted operand): a 64 x 64
// tile of the (Y, X) domain per workgroup, 2 x 2 waves of 8 x 8 lanes, each
// lane owning a 4 x 4 block of cells. An operand contiguous along X is read
// as 4 row vectors, one contiguous along Y as 4 column vectors; the 4 x 4
// block is transposed in registers (it is only a choice of which register
// feeds which cell), so no LDS round trip and no barrier is needed. Every
// vector read and write of a wave covers whole 128-byte lines. Interior
// tiles run without range checks; edge tiles check the domain and masks.
// ---------------------------------------------------------------------------
std::string Gen::gen_tiled() {
    const int X = rank - 1, Y = rank - 2;
    const int64_t NX = k.domain[X], NY = k.domain[Y];
    std::ostringstream b;
    std::vector<int> used(k.leaves.size(), 0);
    for (size_t e = 0; e < k.ex.size(); ++e)
        if (live[e] && k.ex[e].op == RV_BUFFER) used[k.ex[e].leaf] = 1;
    // tile plan: WX x WY waves of 8 x 8 lanes, 4 x 4 cells per lane
    int WX = 2, WY = 2, ORDER = 0;
    sscanf(k.plan_json.c_str(), "\"tile\":[%*d,%*d],\"waves\":[%d,%d],\"order\":%d", &WY, &WX, &ORDER);
    const int TX = 32 * WX, TY = 32 * WY;
    const int64_t GX = (NX + TX - 1) / TX, GY = (NY + TY - 1) / TY;
    b << "  const int t = threadIdx.x, lane = t & 63, w = t >> 6;\n";
    b << "  const " << I << " bid = blockIdx.x;\n";
    switch (ORDER) {
        case 1:  // consecutive workgroups walk Y
            b << "  const " << I << " ty = bid % " << lit(GY) << ", tx = bid / " << lit(GY) << ";\n";
            break;
        case 2:  // diagonal: consecutive workgroups differ in both X and Y
            b << "  const " << I << " tx = bid % " << lit(GX) << ", ty = (bid / " << lit(GX) << " + tx) % " << lit(GY)
              << ";\n";
            break;
        case 3: {  // each XCD (bid % 8 under round-robin dispatch) owns a contiguous range of tiles
            int64_t n = GX * GY;
            if (n % 8 == 0) {
                b << "  const " << I << " sb = (bid & 7) * " << lit(n / 8) << " + (bid >> 3);\n";
                b << "  const " << I << " tx = sb % " << lit(GX) << ", ty = sb / " << lit(GX) << ";\n";
                break;
            }
        }
        // fall through
        default:
            b << "  const " << I << " tx = bid % " << lit(GX) << ", ty = bid / " << lit(GX) << ";\n";
    }
    b << "  const " << I << " X0 = tx * " << TX << ", Y0 = ty * " << TY << ";\n";
    b << "  const " << I << " x = X0 + (w % " << WX << ") * 32 + (lane & 7) * 4;\n";
    b << "  const " << I << " y = Y0 + (w / " << WX << ") * 32 + (lane >> 3) * 4;\n";
    {
        std::string rem = "(" + I + ")blockIdx.z";
        for (int d = Y - 1; d >= 0; --d) {
            b << "  const " << I << " i" << d << " = " << rem << " % " << lit(k.domain[d]) << ";\n";
            if (d > 0) {
                b << "  const " << I << " q" << d << " = " << rem << " / " << lit(k.domain[d]) << ";\n";
                rem = "q" + std::to_string(d);
            }
        }
    }
    auto idx_at = [&](const std::string& yy, const std::string& xx) {
        std::vector<std::string> idx(rank);
        for (int d = 0; d < Y; ++d) idx[d] = fmt("i%d", d);
        idx[Y] = yy;
        idx[X] = xx;
        return idx;
    };
    std::vector<int> all;
    for (int d = 0; d < rank; ++d) all.push_back(d);
    // interior: the whole workgroup tile is inside the domain and every mask
    std::string inter = fmt("X0 + %d <= %s && Y0 + %d <= %s", TX, lit(NX).c_str(), TY, lit(NY).c_str());
    for (size_t l = 0; l < k.leaves.size(); ++l) {
        const Leaf& L = k.leaves[l];
        if (!used[l] || L.zero) continue;
        for (int d = 0; d < rank; ++d) {
            if (!masked(L.v, d)) continue;
            if (d == X)
                inter += fmt(" && X0 >= %s && X0 + %d <= %s", lit(L.v.mask_lo[d]).c_str(), TX, lit(L.v.mask_hi[d]).c_str());
            else if (d == Y)
                inter += fmt(" && Y0 >= %s && Y0 + %d <= %s", lit(L.v.mask_lo[d]).c_str(), TY, lit(L.v.mask_hi[d]).c_str());
            else
                inter += fmt(" && i%d >= %s && i%d < %s", d, lit(L.v.mask_lo[d]).c_str(), d, lit(L.v.mask_hi[d]).c_str());
        }
    }
    b << "  const bool interior = " << inter << ";\n";
    for (int edge = 0; edge < 2; ++edge) {
        b << (edge ? "  else {\n" : "  if (interior) {\n");
        // loads: cell (r, c) of the lane's block is (y + r, x + c). In edge
        // tiles a lane whose 4 x 4 block lies inside the domain and the mask
        // still takes the vector path; only blocks on a boundary go cell by cell.
        for (size_t l = 0; l < k.leaves.size(); ++l) {
            const Leaf& L = k.leaves[l];
            if (!used[l] || L.zero) continue;
            std::string P = pname(L.loc, L.dtype, false);
            std::string V = fmt("l%zu", l);
            const std::string T = st(L.dtype);
            b << "    " << vt(L.dtype) << " " << V << "[4][4];\n";
            const bool along_x = leaf_vec_ok(L, X, 4);
            const bool along_y = !along_x && leaf_vec_ok(L, Y, 4);
            const bool ybcast = L.v.strides[Y] == 0 && !masked(L.v, Y);
            const bool xbcast = L.v.strides[X] == 0 && !masked(L.v, X);
            std::ostringstream vec;
            if (along_x) {
                if (ybcast) {
                    vec << "    { const rv_pack<" << T << ", 4> v = " << vload(L, 4, P + " + " + addr(L.v, idx_at("y", "x")))
                        << ";\n";
                    vec << "      for (int r = 0; r < 4; ++r) for (int c = 0; c < 4; ++c) " << V << "[r][c] = "
                        << ld(L.dtype, "v.v[c]") << "; }\n";
                } else {
                    vec << "    for (int r = 0; r < 4; ++r) { const rv_pack<" << T << ", 4> v = "
                        << vload(L, 4, P + " + " + addr(L.v, idx_at("y + r", "x"))) << ";\n";
                    vec << "      for (int c = 0; c < 4; ++c) " << V << "[r][c] = " << ld(L.dtype, "v.v[c]") << "; }\n";
                }
            } else if (along_y) {
                if (xbcast) {
                    vec << "    { const rv_pack<" << T << ", 4> v = " << vload(L, 4, P + " + " + addr(L.v, idx_at("y", "x")))
                        << ";\n";
                    vec << "      for (int r = 0; r < 4; ++r) for (int c = 0; c < 4; ++c) " << V << "[r][c] = "
                        << ld(L.dtype, "v.v[r]") << "; }\n";
                } else {
                    vec << "    for (int c = 0; c < 4; ++c) { const rv_pack<" << T << ", 4> v = "
                        << vload(L, 4, P + " + " + addr(L.v, idx_at("y", "x + c"))) << ";\n";
                    vec << "      for (int r = 0; r < 4; ++r) " << V << "[r][c] = " << ld(L.dtype, "v.v[r]") << "; }\n";
                }
            }
            std::ostringstream sc;
            sc << "    for (int r = 0; r < 4; ++r) for (int c = 0; c < 4; ++c) {\n";
            sc << "      const " << I << " yy = y + r, xx = x + c;\n";
            auto idq = idx_at("yy", "xx");
            std::string mc = edge ? mask_cond(L.v, idq, all) : "";
            std::string cond = edge ? fmt("yy < %s && xx < %s", lit(NY).c_str(), lit(NX).c_str()) +
                                          (mc.empty() ? "" : " && " + mc)
                                    : "";
            sc << "      " << V << "[r][c] = " << (cond.empty() ? "" : "(" + cond + ") ? ")
               << ld(L.dtype, P + "[" + addr(L.v, idq) + "]") << (cond.empty() ? "" : " : " + zero_of(L.dtype))
               << ";\n    }\n";
            if (!along_x && !along_y) {
                b << sc.str();
            } else if (!edge) {
                b << vec.str();
            } else {
                // the block is inside the domain and the leaf's mask
                std::string in = fmt("y + 4 <= %s && x + 4 <= %s", lit(NY).c_str(), lit(NX).c_str());
                for (int d = 0; d < rank; ++d) {
                    if (!masked(L.v, d)) continue;
                    if (d == X)
                        in += fmt(" && x >= %s && x + 4 <= %s", lit(L.v.mask_lo[d]).c_str(), lit(L.v.mask_hi[d]).c_str());
                    else if (d == Y)
                        in += fmt(" && y >= %s && y + 4 <= %s", lit(L.v.mask_lo[d]).c_str(), lit(L.v.mask_hi[d]).c_str());
                    else
                        in += fmt(" && i%d >= %s && i%d < %s", d, lit(L.v.mask_lo[d]).c_str(), d,
                                  lit(L.v.mask_hi[d]).c_str());
                }
                b << "    if (" << in << ") {\n" << vec.str() << "    } else {\n" << sc.str() << "    }\n";
            }
        }
        for (size_t e = 0; e < k.ex.size(); ++e) {
            if (!live[e]) continue;
            const Ex& x = k.ex[e];
            b << "    " << vt(x.dtype) << " e" << e << "[4][4];\n    for (int r = 0; r < 4; ++r) for (int c = 0; c < 4; ++c) e"
              << e << "[r][c] = ";
            if (x.op == RV_BUFFER) {
                if (k.leaves[x.leaf].zero)
                    b << zero_of(x.dtype);
                else
                    b << "l" << x.leaf << "[r][c]";
            } else if (x.op == RV_CONST) {
                b << const_lit(x.dtype, x.cval);
            } else {
                auto E = [&](int i) { return i < 0 ? std::string() : fmt("e%d[r][c]", i); };
                b << op_code(k, x, E(x.a), E(x.b), E(x.c));
            }
            b << ";\n";
        }
        for (const Store& s : k.stores) {
            std::string P = pname(s.loc, s.dtype, true);
            bool vec = s.v.strides[X] == 1 && s.v.offset % 4 == 0;
            for (int d = 0; d < X; ++d)
                if (k.domain[d] > 1 && s.v.strides[d] % 4) vec = false;
            if (vec) {
                if (edge) b << "    if (y + 4 <= " << lit(NY) << " && x + 4 <= " << lit(NX) << ") {\n";
                b << "    for (int r = 0; r < 4; ++r) { rv_pack<" << st(s.dtype) << ", 4> v;\n";
                b << "      for (int c = 0; c < 4; ++c) v.v[c] = " << sv(s.dtype, fmt("e%d[r][c]", s.ex)) << ";\n";
                b << "      " << vstore(s.dtype, 4, P + " + " + addr(s.v, idx_at("y + r", "x")), "v") << "; }\n";
                if (edge) {
                    b << "    } else\n";
                    b << "    for (int r = 0; r < 4; ++r) for (int c = 0; c < 4; ++c) {\n";
                    b << "      const " << I << " yy = y + r, xx = x + c;\n";
                    b << "      if (yy < " << lit(NY) << " && xx < " << lit(NX) << ") " << P << "["
                      << addr(s.v, idx_at("yy", "xx")) << "] = " << sv(s.dtype, fmt("e%d[r][c]", s.ex)) << ";\n    }\n";
                }
            } else {
                b << "    for (int r = 0; r < 4; ++r) for (int c = 0; c < 4; ++c) {\n";
                b << "      const " << I << " yy = y + r, xx = x + c;\n";
                b << "      " << (edge ? fmt("if (yy < %s && xx < %s) ", lit(NY).c_str(), lit(NX).c_str()) : "") << P
                  << "[" << addr(s.v, idx_at("yy", "xx")) << "] = " << sv(s.dtype, fmt("e%d[r][c]", s.ex)) << ";\n    }\n";
            }
        }
        b << "  }\n";
    }
    return b.str();
}

// ---------------------------------------------------------------------------
// ROW plan: T threads cooperate on one row (RPW rows per workgroup); a thread
// keeps its E = NV * VW cells of every full-row value in registers, so the
// row is read once. Reductions fold a thread's cells, then a butterfly over
// the row's lanes, then (T > 64) the waves' totals in a fixed order in LDS.
// Row-constant operands (weights) are read once per workgroup.
// ---------------------------------------------------------------------------
std::string Gen::gen_row() {
    std::vector<int> rd, kd;
    for (int d = 0; d < rank; ++d) ((k.rdims >> d) & 1u ? rd : kd).push_back(d);
    int64_t NR = 1, NK = 1;
    for (int d : rd) NR *= k.domain[d];
    for (int d : kd) NK *= k.domain[d];
    // plan values (mirrors lower.cpp)
    int T = 0, VW = 0;
    sscanf(k.plan_json.c_str(), "\"threads_per_row\":%d,\"rows_per_block\":%*d,\"vec\":%d", &T, &VW);
    const int RPW = (int)k.block[0] / T;
    const int NV = (int)((NR + (int64_t)T * VW - 1) / ((int64_t)T * VW));
    const int E = NV * VW;
    const bool ragged = NR % ((int64_t)T * VW) != 0;
    const int W = T > 64 ? T / 64 : 1;
    const int nred_ = [&] {
        int n = 0;
        for (size_t e = 0; e < k.ex.size(); ++e)
            if (live[e] && (k.ex[e].op == RV_SUM || k.ex[e].op == RV_MAX)) ++n;
        return n;
    }();
    const bool single = rd.size() == 1;
    const int R = single ? rd[0] : -1;
    // stat flags on lowered views
    std::vector<char> stat(k.ex.size(), 0);
    for (size_t e = 0; e < k.ex.size(); ++e) {
        const Ex& x = k.ex[e];
        if (x.op == RV_BUFFER) {
            const Leaf& L = k.leaves[x.leaf];
            bool s = true;
            for (int d : rd)
                if (!L.zero && (L.v.strides[d] != 0 || masked(L.v, d))) s = false;
            stat[e] = s;
        } else if (x.op == RV_CONST || x.op == RV_SUM || x.op == RV_MAX) {
            stat[e] = 1;
        } else {
            stat[e] = (x.a < 0 || stat[x.a]) && (x.b < 0 || stat[x.b]) && (x.c < 0 || stat[x.c]);
        }
    }
    // hoisted leaves: full along the row, constant across rows, unmasked across rows
    auto hoistable = [&](const Leaf& L) {
        for (int d : kd)
            if (L.v.strides[d] != 0 || masked(L.v, d)) return false;
        return true;
    };
    std::ostringstream b;
    b << "  const int t = threadIdx.x, lt = t % " << T << ", lr = t / " << T << ";\n";
    bool wide_red = false;  // a float64 or int reduce: its partials travel through LDS as double
    for (size_t e = 0; e < k.ex.size(); ++e)
        if (live[e] && (k.ex[e].op == RV_SUM || k.ex[e].op == RV_MAX) && !(k.ex[e].dtype == RV_F32 || is_half(k.ex[e].dtype)))
            wide_red = true;
    if (T > 64 && nred_)
        b << "  __shared__ " << (wide_red ? "double" : "float") << " red[" << nred_ << "][" << RPW << "][" << W << "];\n";
    // element index helpers: n(v, i) = (v * T + lt) * VW + i
    auto nexpr = [&](const std::string& v, const std::string& i) {
        return fmt("(((%s) * %d + lt) * %d + (%s))", v.c_str(), T, VW, i.c_str());
    };
    // reduced-dim index expressions from a flat in-row index n
    auto red_idx = [&](std::vector<std::string>& idx, const std::string& n) {
        if (single) {
            idx[R] = n;
            return;
        }
        std::string rem = n;
        for (size_t j = rd.size(); j-- > 0;) {
            int d = rd[j];
            idx[d] = j ? fmt("((%s) %% %s)", rem.c_str(), lit(k.domain[d]).c_str()) : rem;
            if (j) rem = fmt("((%s) / %s)", rem.c_str(), lit(k.domain[d]).c_str());
        }
    };
    std::vector<int> used(k.leaves.size(), 0);
    for (size_t e = 0; e < k.ex.size(); ++e)
        if (live[e] && k.ex[e].op == RV_BUFFER) used[k.ex[e].leaf] = 1;
    auto emit_full_load = [&](std::ostringstream& s, int l, const std::string& rowok, const std::vector<std::string>& kidx,
                              const std::string& V, bool raw) {
        const Leaf& L = k.leaves[l];
        std::string P = pname(L.loc, L.dtype, false);
        // raw: keep the storage type in registers (hoisted weights: half the
        // VGPRs for 2-byte dtypes), widened where they are used
        auto ld = [&](int dt, const std::string& e) { return raw ? e : rv::ld(dt, e); };
        s << "    " << (raw ? st(L.dtype) : vt(L.dtype)) << " " << V << "[" << E << "];\n";
        s << "    for (int v = 0; v < " << NV << "; ++v) {\n";
        s << "      const " << I << " n0 = " << nexpr("v", "0") << ";\n";
        std::vector<std::string> idx = kidx;
        bool vec = single && leaf_vec_ok(L, R, VW);
        if (vec) {
            idx[R] = "n0";
            std::string mc = masked(L.v, R) ? fmt(" && n0 >= %s && n0 + %d <= %s", lit(L.v.mask_lo[R]).c_str(), VW,
                                                  lit(L.v.mask_hi[R]).c_str())
                                            : "";
            std::string rg = ragged ? fmt(" && n0 + %d <= %s", VW, lit(NR).c_str()) : "";
            s << "      if (" << rowok << mc << rg << ") {\n";
            s << "        const rv_pack<" << st(L.dtype) << ", " << VW << "> p = "
              << (raw ? "rv_ldv<" + st(L.dtype) + ", " + std::to_string(VW) + ">(" + P + " + " + addr(L.v, idx) + ")"
                      : vload(L, VW, P + " + " + addr(L.v, idx)))
              << ";\n";
            s << "        for (int i = 0; i < " << VW << "; ++i) " << V << "[v * " << VW << " + i] = " << ld(L.dtype, "p.v[i]")
              << ";\n      } else\n";
        }
        s << "      for (int i = 0; i < " << VW << "; ++i) {\n";
        s << "        const " << I << " n = n0 + i;\n";
        red_idx(idx, "n");
        std::string mc = mask_cond(L.v, idx, rd);
        s << "        " << V << "[v * " << VW << " + i] = (" << rowok << " && n < " << lit(NR) << (mc.empty() ? "" : " && " + mc)
          << ") ? " << ld(L.dtype, P + "[" + addr(L.v, idx) + "]") << " : " << (raw ? "0" : zero_of(L.dtype)) << ";\n";
        s << "      }\n    }\n";
    };
    // hoisted loads
    std::vector<int> hoisted(k.leaves.size(), 0);
    {
        std::vector<std::string> kidx(rank);
        for (size_t l = 0; l < k.leaves.size(); ++l) {
            const Leaf& L = k.leaves[l];
            if (!used[l] || L.zero) continue;
            bool full = false;
            for (int d : rd)
                if (L.v.strides[d] != 0 || masked(L.v, d)) full = true;
            if (full && hoistable(L)) {
                hoisted[l] = 1;
                std::ostringstream s;
                emit_full_load(s, (int)l, "true", kidx, fmt("h%zu", l), true);
                b << s.str();
            }
        }
    }
    const int64_t NRG = (NK + RPW - 1) / RPW;
    // prefetch (persistent grid): a streamed leaf whose row is one run of
    // aligned vectors is loaded one row group ahead into registers of its
    // storage type, so its next row is in flight while this one is reduced
    const bool pf = k.plan_json.find("\"prefetch\":1") != std::string::npos && single && !ragged;
    std::vector<int> pfl(k.leaves.size(), 0);
    if (pf)
        for (size_t l = 0; l < k.leaves.size(); ++l) {
            const Leaf& L = k.leaves[l];
            if (!used[l] || L.zero || hoisted[l] || masked(L.v, R) || !leaf_vec_ok(L, R, VW)) continue;
            if (L.v.strides[R] == 0) continue;
            pfl[l] = 1;
        }
    // row index variables r<sfx>, rv<sfx>, i<d><sfx> of row group rgx
    auto row_vars = [&](std::ostringstream& s, const std::string& sfx, const std::string& rgx,
                        const std::string& ind) {
        std::vector<std::string> kx(rank);
        s << ind << "const " << I << " r" << sfx << " = (" << rgx << ") * " << RPW << " + lr;\n";
        s << ind << "const bool rv" << sfx << " = (" << rgx << ") < " << lit(NRG) << " && r" << sfx << " < " << lit(NK)
          << ";\n";
        std::string rem = "r" + sfx;
        for (size_t j = kd.size(); j-- > 0;) {
            int d = kd[j];
            s << ind << "const " << I << " i" << d << sfx << " = "
              << (j ? fmt("%s %% %s", rem.c_str(), lit(k.domain[d]).c_str()) : rem) << ";\n";
            kx[d] = fmt("i%d%s", d, sfx.c_str());
            if (j) {
                s << ind << "const " << I << " q" << d << sfx << " = " << rem << " / " << lit(k.domain[d]) << ";\n";
                rem = fmt("q%d%s", d, sfx.c_str());
            }
        }
        return kx;
    };
    auto emit_pf_loads = [&](std::ostringstream& s, const std::string& sfx, const std::vector<std::string>& kx,
                             const std::string& ind) {
        for (size_t l = 0; l < k.leaves.size(); ++l) {
            if (!pfl[l]) continue;
            const Leaf& L = k.leaves[l];
            std::string kc = mask_cond(L.v, kx, kd);
            std::string rowok = "rv" + sfx + (kc.empty() ? std::string() : " && " + kc);
            std::vector<std::string> idx = kx;
            idx[R] = "n0";
            s << ind << "for (int v = 0; v < " << NV << "; ++v) {\n";
            s << ind << "  const " << I << " n0 = " << nexpr("v", "0") << ";\n";
            s << ind << "  if (" << rowok << ") f" << l << "[v] = " << vload(L, VW, pname(L.loc, L.dtype, false) + " + " + addr(L.v, idx))
              << ";\n";
            s << ind << "  else f" << l << "[v] = rv_pack<" << st(L.dtype) << ", " << VW << ">{};\n";
            s << ind << "}\n";
        }
    };
    bool any_pf = false;
    for (int x : pfl) any_pf = any_pf || x;
    if (any_pf) {
        for (size_t l = 0; l < k.leaves.size(); ++l)
            if (pfl[l]) b << "  rv_pack<" << st(k.leaves[l].dtype) << ", " << VW << "> f" << l << "[" << NV << "];\n";
        b << "  {\n";
        std::ostringstream s;
        auto kx = row_vars(s, "", "blockIdx.x", "    ");
        emit_pf_loads(s, "", kx, "    ");
        b << s.str() << "  }\n";
    }
    b << "  for (" << I << " rg = blockIdx.x; rg < " << lit(NRG) << "; rg += gridDim.x) {\n";
    if (T > 64 && nred_) b << "    rv_lds_barrier();\n";
    b << "    const " << I << " r = rg * " << RPW << " + lr;\n";
    b << "    const bool rv = r < " << lit(NK) << ";\n";
    std::vector<std::string> kidx(rank);
    {
        std::string rem = "r";
        for (size_t j = kd.size(); j-- > 0;) {
            int d = kd[j];
            b << "    const " << I << " i" << d << " = " << (j ? fmt("%s %% %s", rem.c_str(), lit(k.domain[d]).c_str()) : rem)
              << ";\n";
            kidx[d] = fmt("i%d", d);
            if (j) {
                b << "    const " << I << " q" << d << " = " << rem << " / " << lit(k.domain[d]) << ";\n";
                rem = fmt("q%d", d);
            }
        }
    }
    if (any_pf) {
        for (size_t l = 0; l < k.leaves.size(); ++l)
            if (pfl[l]) {
                b << "    rv_pack<" << st(k.leaves[l].dtype) << ", " << VW << "> c" << l << "[" << NV << "];\n";
                b << "    for (int v = 0; v < " << NV << "; ++v) c" << l << "[v] = f" << l << "[v];\n";
            }
        b << "    {\n";
        std::ostringstream s;
        auto kx = row_vars(s, "n", "rg + gridDim.x", "      ");
        emit_pf_loads(s, "n", kx, "      ");
        b << s.str() << "    }\n";
    }
    int red_slot = 0;
    // value of ex i at in-thread position q (a scalar for row-constant values)
    auto fullv = [&](int i, const std::string& q) -> std::string {
        if (i < 0) return "";
        const Ex& x = k.ex[i];
        if (x.op == RV_BUFFER && !k.leaves[x.leaf].zero && hoisted[x.leaf])
            return ld(x.dtype, fmt("h%d[%s]", x.leaf, q.c_str()));
        return stat[i] ? fmt("e%d", i) : fmt("e%d[%s]", i, q.c_str());
    };
    for (size_t e = 0; e < k.ex.size(); ++e) {
        if (!live[e]) continue;
        const Ex& x = k.ex[e];
        std::string V = fmt("e%zu", e);
        if (x.op == RV_BUFFER) {
            const Leaf& L = k.leaves[x.leaf];
            if (L.zero) {
                b << "    const " << vt(x.dtype) << " " << V << " = " << zero_of(x.dtype) << ";\n";
                stat[e] = 1;
                continue;
            }
            if (hoisted[x.leaf]) continue;  // read as h<leaf>[q] where used
            if (pfl[x.leaf]) {
                b << "    " << vt(x.dtype) << " " << V << "[" << E << "];\n";
                b << "    for (int v = 0; v < " << NV << "; ++v)\n      for (int i = 0; i < " << VW << "; ++i) " << V
                  << "[v * " << VW << " + i] = " << ld(L.dtype, fmt("c%d[v].v[i]", x.leaf)) << ";\n";
                continue;
            }
            std::string kc = mask_cond(L.v, kidx, kd);
            std::string rowok = "rv" + (kc.empty() ? std::string() : " && " + kc);
            if (stat[e]) {
                std::string P = pname(L.loc, L.dtype, false);
                b << "    const " << vt(x.dtype) << " " << V << " = (" << rowok << ") ? "
                  << ld(L.dtype, P + "[" + addr(L.v, kidx) + "]") << " : " << zero_of(x.dtype) << ";\n";
            } else {
                std::ostringstream s;
                emit_full_load(s, x.leaf, rowok, kidx, V, false);
                b << s.str();
            }
            continue;
        }
        if (x.op == RV_CONST) {
            b << "    const " << vt(x.dtype) << " " << V << " = " << const_lit(x.dtype, x.cval) << ";\n";
            continue;
        }
        auto opnd = [&](int i, const std::string& q) -> std::string { return fullv(i, q); };
        if (x.op == RV_SUM || x.op == RV_MAX) {
            const bool sum = x.op == RV_SUM;
            const RedType rt(x.op, x.dtype);
            b << "    " << vt(x.dtype) << " " << V << ";\n    {\n";
            b << "      " << rt.t << " acc = " << rt.ident << ";\n";
            b << "      for (int q = 0; q < " << E << "; ++q) {\n";
            std::string val = opnd(x.a, "q");
            if (ragged)
                b << "        if (" << nexpr("q / " + std::to_string(VW), "q % " + std::to_string(VW)) << " < " << lit(NR)
                  << ") ";
            else
                b << "        ";
            b << "acc = " << rt.fold("acc", val) << ";\n      }\n";
            int g = std::min(T, 64);
            b << "      acc = rv_group_" << (sum ? "sum" : "max") << "<" << g << ">(acc);\n";
            if (T > 64) {
                b << "      if ((t & 63) == 0) red[" << red_slot << "][lr][lt >> 6] = acc;\n      rv_lds_barrier();\n";
                b << "      acc = (" << rt.t << ")red[" << red_slot << "][lr][0];\n";
                for (int w = 1; w < W; ++w)
                    b << "      acc = " << rt.fold("acc", fmt("(%s)red[%d][lr][%d]", rt.t.c_str(), red_slot, w)) << ";\n";
                ++red_slot;
            }
            b << "      " << V << " = " << rt.result(x.dtype, "acc") << ";\n    }\n";
            continue;
        }
        if (stat[e]) {
            b << "    const " << vt(x.dtype) << " " << V << " = " << op_code(k, x, opnd(x.a, ""), opnd(x.b, ""), opnd(x.c, ""))
              << ";\n";
        } else {
            b << "    " << vt(x.dtype) << " " << V << "[" << E << "];\n";
            b << "    for (int q = 0; q < " << E << "; ++q) " << V << "[q] = "
              << op_code(k, x, opnd(x.a, "q"), opnd(x.b, "q"), opnd(x.c, "q")) << ";\n";
        }
    }
    for (const Store& s : k.stores) {
        std::string P = pname(s.loc, s.dtype, true);
        bool sstat = true;
        for (int d : rd)
            if (s.v.strides[d] != 0) sstat = false;
        if (sstat) {
            std::string val = fullv(s.ex, "0");
            b << "    if (lt == 0 && rv) " << P << "[" << addr(s.v, kidx) << "] = " << sv(s.dtype, val) << ";\n";
            continue;
        }
        std::string val = fullv(s.ex, fmt("v * %d + i", VW));
        b << "    for (int v = 0; v < " << NV << "; ++v) {\n";
        b << "      const " << I << " n0 = " << nexpr("v", "0") << ";\n";
        std::vector<std::string> idx = kidx;
        bool vec = single && s.v.strides[R] == 1 && s.v.offset % VW == 0;
        for (int d : kd)
            if (k.domain[d] > 1 && s.v.strides[d] % VW) vec = false;
        if (vec) {
            idx[R] = "n0";
            std::string rg = ragged ? fmt(" && n0 + %d <= %s", VW, lit(NR).c_str()) : "";
            b << "      if (rv" << rg << ") {\n        rv_pack<" << st(s.dtype) << ", " << VW << "> p;\n";
            b << "        for (int i = 0; i < " << VW << "; ++i) p.v[i] = " << sv(s.dtype, val) << ";\n";
            b << "        " << vstore(s.dtype, VW, P + " + " + addr(s.v, idx), "p") << ";\n";
            b << "      } else\n";
        }
        b << "      for (int i = 0; i < " << VW << "; ++i) {\n        const " << I << " n = n0 + i;\n";
        red_idx(idx, "n");
        b << "        if (rv && n < " << lit(NR) << ") " << P << "[" << addr(s.v, idx) << "] = " << sv(s.dtype, val) << ";\n";
        b << "      }\n    }\n";
    }
    b << "  }\n";
    return b.str();
}

// ---------------------------------------------------------------------------
// ROW, streaming plan: for rows too long to keep in registers. The row is
// walked in chunks of T * VW * U cells (each lane U vectors of VW), once per
// reduce and once more for the full-row outputs, with O(1) state per lane;
// each reduce's result is a row constant for the passes after it. A MAX and
// a SUM of EXP(X - MAX(X)) share one pass through the online recurrence
// (Tiki README, "Write the attention kernel at the algorithm level":
// running maximum and denominator, the denominator rescaled by
// exp(m_old - m_new) whenever the maximum grows),
// so softmax reads its row twice instead of three times. A range whose
// values are all -inf so far keeps m = -inf and adds nothing, so masked
// entries never produce -inf - (-inf).
// ---------------------------------------------------------------------------
std::string Gen::gen_row_stream() {
    std::vector<int> rd, kd;
    for (int d = 0; d < rank; ++d) ((k.rdims >> d) & 1u ? rd : kd).push_back(d);
    int64_t NR = 1, NK = 1;
    for (int d : rd) NR *= k.domain[d];
    for (int d : kd) NK *= k.domain[d];
    int T = 0, VW = 0, U = 4;
    sscanf(k.plan_json.c_str(), "\"threads_per_row\":%d,\"rows_per_block\":%*d,\"vec\":%d", &T, &VW);
    {
        size_t at = k.plan_json.find("\"unroll\":");
        if (at != std::string::npos) sscanf(k.plan_json.c_str() + at, "\"unroll\":%d", &U);
    }
    // a split reduce: workgroup (row, piece) folds chunks
    // [piece * CPP, (piece + 1) * CPP) and writes its raw total to the
    // partials ([row][piece]) instead of finishing the row
    const bool split = k.cls == KClass::SPLIT;
    int64_t SP = 1, CPP = 0;
    if (split) {
        size_t at = k.plan_json.find("\"pieces\":");
        if (at != std::string::npos) sscanf(k.plan_json.c_str() + at, "\"pieces\":%lld,\"chunks_per_piece\":%lld",
                                            (long long*)&SP, (long long*)&CPP);
        if (SP < 1 || CPP < 1) fail(RV_E_INVALID, "internal: split plan without pieces");
    }
    const int RPW = (int)k.block[0] / T;
    const int W = T > 64 ? T / 64 : 1;
    const int E = VW * U;
    const int64_t CH = (int64_t)T * E;
    const int64_t NCH = (NR + CH - 1) / CH;
    const bool ragged = NR % CH != 0;
    const bool single = rd.size() == 1;
    const int R = single ? rd[0] : -1;
    const auto pairs = online_softmax_pairs(k);
    std::vector<int> pair_of(k.ex.size(), -1);  // max -> sum, sum -> max
    for (auto& pr : pairs) pair_of[pr.first] = pr.second, pair_of[pr.second] = pr.first;
    // row-constant values
    std::vector<char> stat(k.ex.size(), 0);
    for (size_t e = 0; e < k.ex.size(); ++e) {
        const Ex& x = k.ex[e];
        if (x.op == RV_BUFFER) {
            const Leaf& L = k.leaves[x.leaf];
            bool st_ = true;
            for (int d : rd)
                if (!L.zero && (L.v.strides[d] != 0 || masked(L.v, d))) st_ = false;
            stat[e] = st_;
        } else if (x.op == RV_CONST || x.op == RV_SUM || x.op == RV_MAX) {
            stat[e] = 1;
        } else {
            stat[e] = (x.a < 0 || stat[x.a]) && (x.b < 0 || stat[x.b]) && (x.c < 0 || stat[x.c]);
        }
    }
    // passes: one per reduce, a MAX and its paired SUM together
    std::vector<std::vector<int>> passes;
    for (size_t e = 0; e < k.ex.size(); ++e) {
        if (!live[e] || (k.ex[e].op != RV_SUM && k.ex[e].op != RV_MAX)) continue;
        if (k.ex[e].op == RV_SUM && pair_of[e] >= 0) continue;  // folded with its MAX
        if (k.ex[e].op == RV_MAX && pair_of[e] >= 0)
            passes.push_back({(int)e, pair_of[e]});
        else
            passes.push_back({(int)e});
    }
    const int nslots = (int)passes.size() + (int)pairs.size();
    std::ostringstream b;
    b << "  const int t = threadIdx.x, lt = t % " << T << ", lr = t / " << T << ";\n";
    bool wide_red = false;  // a float64 or int reduce: its partials travel through LDS as double
    for (size_t e = 0; e < k.ex.size(); ++e)
        if (live[e] && (k.ex[e].op == RV_SUM || k.ex[e].op == RV_MAX) && !(k.ex[e].dtype == RV_F32 || is_half(k.ex[e].dtype)))
            wide_red = true;
    if (T > 64 && nslots)
        b << "  __shared__ " << (wide_red ? "double" : "float") << " red[" << nslots << "][" << RPW << "][" << W << "];\n";
    auto nexpr = [&](const std::string& v, const std::string& i) {
        return fmt("(cb + ((%s) * %d + lt) * %d + (%s))", v.c_str(), T, VW, i.c_str());
    };
    auto red_idx = [&](std::vector<std::string>& idx, const std::string& n) {
        if (single) {
            idx[R] = n;
            return;
        }
        std::string rem = n;
        for (size_t j = rd.size(); j-- > 0;) {
            int d = rd[j];
            idx[d] = j ? fmt("((%s) %% %s)", rem.c_str(), lit(k.domain[d]).c_str()) : rem;
            if (j) rem = fmt("((%s) / %s)", rem.c_str(), lit(k.domain[d]).c_str());
        }
    };
    const std::string inrow = fmt("%s < %s", nexpr("q / " + std::to_string(VW), "q % " + std::to_string(VW)).c_str(),
                                  lit(NR).c_str());
    const int64_t NRG = (NK + RPW - 1) / RPW;
    if (split) {
        b << "  {\n    const " << I << " rg = (" << I << ")blockIdx.x / " << lit(SP) << ";\n";
        b << "    const " << I << " piece = (" << I << ")blockIdx.x % " << lit(SP) << ";\n";
        b << "    const " << I << " c0 = piece * " << lit(CPP) << ";\n";
        b << "    const " << I << " c1 = c0 + " << lit(CPP) << " < " << lit(NCH) << " ? c0 + " << lit(CPP) << " : "
          << lit(NCH) << ";\n";
    } else {
        b << "  for (" << I << " rg = blockIdx.x; rg < " << lit(NRG) << "; rg += gridDim.x) {\n";
    }
    if (T > 64 && nslots) b << "    rv_lds_barrier();\n";
    b << "    const " << I << " r = rg * " << RPW << " + lr;\n";
    b << "    const bool rv = r < " << lit(NK) << ";\n";
    std::vector<std::string> kidx(rank);
    {
        std::string rem = "r";
        for (size_t j = kd.size(); j-- > 0;) {
            int d = kd[j];
            b << "    const " << I << " i" << d << " = " << (j ? fmt("%s %% %s", rem.c_str(), lit(k.domain[d]).c_str()) : rem)
              << ";\n";
            kidx[d] = fmt("i%d", d);
            if (j) {
                b << "    const " << I << " q" << d << " = " << rem << " / " << lit(k.domain[d]) << ";\n";
                rem = fmt("q%d", d);
            }
        }
    }
    auto V = [&](int i, const std::string& q) -> std::string {
        return stat[i] ? fmt("e%d", i) : fmt("e%d[%s]", i, q.c_str());
    };
    // row constants whose inputs are ready
    std::vector<char> done(k.ex.size(), 0);
    auto emit_ready = [&](const std::string& ind) {
        for (size_t e = 0; e < k.ex.size(); ++e) {
            const Ex& x = k.ex[e];
            if (!live[e] || !stat[e] || done[e] || x.op == RV_SUM || x.op == RV_MAX) continue;
            if ((x.a >= 0 && !done[x.a]) || (x.b >= 0 && !done[x.b]) || (x.c >= 0 && !done[x.c])) continue;
            std::string Vn = fmt("e%zu", e);
            if (x.op == RV_BUFFER) {
                const Leaf& L = k.leaves[x.leaf];
                if (L.zero) {
                    b << ind << "const " << vt(x.dtype) << " " << Vn << " = " << zero_of(x.dtype) << ";\n";
                } else {
                    std::string kc = mask_cond(L.v, kidx, kd);
                    std::string rowok = "rv" + (kc.empty() ? std::string() : " && " + kc);
                    b << ind << "const " << vt(x.dtype) << " " << Vn << " = (" << rowok << ") ? "
                      << ld(L.dtype, pname(L.loc, L.dtype, false) + "[" + addr(L.v, kidx) + "]") << " : "
                      << zero_of(x.dtype) << ";\n";
                }
            } else if (x.op == RV_CONST) {
                b << ind << "const " << vt(x.dtype) << " " << Vn << " = " << const_lit(x.dtype, x.cval) << ";\n";
            } else {
                b << ind << "const " << vt(x.dtype) << " " << Vn << " = "
                  << op_code(k, x, V(x.a, ""), x.b >= 0 ? V(x.b, "") : "", x.c >= 0 ? V(x.c, "") : "") << ";\n";
            }
            done[e] = 1;
        }
    };
    // the full-row values a set of roots needs, in order
    auto needed = [&](const std::vector<int>& roots) {
        std::vector<char> need(k.ex.size(), 0);
        std::function<void(int)> go = [&](int e) {
            if (e < 0 || need[e] || stat[e]) return;
            need[e] = 1;
            go(k.ex[e].a), go(k.ex[e].b), go(k.ex[e].c);
        };
        for (int r0 : roots) go(r0);
        return need;
    };
    // one chunk's full-row values (E cells per lane). Loads before the last
    // pass are plain (cacheable): the row is read again by a later pass.
    auto emit_chunk = [&](const std::vector<char>& need, const std::string& ind, bool last) {
        for (size_t e = 0; e < k.ex.size(); ++e) {
            if (!need[e]) continue;
            const Ex& x = k.ex[e];
            std::string Vn = fmt("e%zu", e);
            if (x.op == RV_BUFFER) {
                const Leaf& L = k.leaves[x.leaf];
                std::string P = pname(L.loc, L.dtype, false);
                std::string kc = mask_cond(L.v, kidx, kd);
                std::string rowok = "rv" + (kc.empty() ? std::string() : " && " + kc);
                b << ind << vt(x.dtype) << " " << Vn << "[" << E << "];\n";
                b << ind << "for (int v = 0; v < " << U << "; ++v) {\n";
                b << ind << "  const " << I << " n0 = " << nexpr("v", "0") << ";\n";
                std::vector<std::string> idx = kidx;
                if (single && leaf_vec_ok(L, R, VW)) {
                    idx[R] = "n0";
                    std::string mc = masked(L.v, R) ? fmt(" && n0 >= %s && n0 + %d <= %s", lit(L.v.mask_lo[R]).c_str(), VW,
                                                          lit(L.v.mask_hi[R]).c_str())
                                                    : "";
                    b << ind << "  if (" << rowok << mc << " && n0 + " << VW << " <= " << lit(NR) << ") {\n";
                    const std::string ptr = P + " + " + addr(L.v, idx);
                    b << ind << "    const rv_pack<" << st(L.dtype) << ", " << VW << "> p = "
                      << (last ? vload(L, VW, ptr) : "rv_ldv<" + st(L.dtype) + ", " + std::to_string(VW) + ">(" + ptr + ")")
                      << ";\n";
                    b << ind << "    for (int i = 0; i < " << VW << "; ++i) " << Vn << "[v * " << VW << " + i] = " << ld(L.dtype, "p.v[i]")
                      << ";\n";
                    b << ind << "  } else\n";
                }
                b << ind << "  for (int i = 0; i < " << VW << "; ++i) {\n";
                b << ind << "    const " << I << " n = n0 + i;\n";
                red_idx(idx, "n");
                std::string mc = mask_cond(L.v, idx, rd);
                b << ind << "    " << Vn << "[v * " << VW << " + i] = (" << rowok << " && n < " << lit(NR)
                  << (mc.empty() ? "" : " && " + mc) << ") ? " << ld(L.dtype, P + "[" + addr(L.v, idx) + "]") << " : "
                  << zero_of(L.dtype == RV_BF16 || L.dtype == RV_F16 ? RV_F32 : L.dtype) << ";\n";
                b << ind << "  }\n" << ind << "}\n";
                continue;
            }
            b << ind << vt(x.dtype) << " " << Vn << "[" << E << "];\n";
            b << ind << "for (int q = 0; q < " << E << "; ++q) " << Vn << "[q] = "
              << op_code(k, x, V(x.a, "q"), x.b >= 0 ? V(x.b, "q") : "", x.c >= 0 ? V(x.c, "q") : "") << ";\n";
        }
    };
    const std::string guard = ragged ? "if (" + inrow + ") " : "";
    int slot = 0;
    emit_ready("    ");
    for (const auto& pass : passes) {
        const int r0 = pass[0];
        const Ex& R0 = k.ex[r0];
        const bool online = pass.size() == 2;
        // operand of the fold: the MAX's operand X for the online pass
        const int X = R0.a;
        b << "    // pass: " << (online ? "online MAX + SUM(EXP(x - max))" : (R0.op == RV_SUM ? "SUM" : "MAX")) << "\n";
        if (online)
            b << "    float om = -__builtin_inff(), ol = 0.0f;\n";
        else
            b << "    " << RedType(R0.op, R0.dtype).t << " acc" << r0 << " = " << RedType(R0.op, R0.dtype).ident << ";\n";
        if (split)
            b << "    for (" << I << " c = c0; c < c1; ++c) {\n";
        else
            b << "    for (" << I << " c = 0; c < " << lit(NCH) << "; ++c) {\n";
        b << "      const " << I << " cb = c * " << lit(CH) << ";\n";
        emit_chunk(needed({X}), "      ", split);
        const std::string xv = V(X, "q");
        if (online) {
            b << "      float cm = -__builtin_inff();\n";
            b << "      for (int q = 0; q < " << E << "; ++q) " << guard << "cm = rv_maxf(cm, " << xv << ");\n";
            b << "      const float mn = rv_maxf(om, cm);\n";
            b << "      const float alpha = (om == mn) ? 1.0f : expf(om - mn);\n";
            b << "      float ps = 0.0f;\n";
            b << "      if (mn != -__builtin_inff())\n";
            b << "        for (int q = 0; q < " << E << "; ++q) " << guard << "ps = ps + expf(" << xv << " + (-mn));\n";
            b << "      ol = ol * alpha + ps;\n      om = mn;\n";
        } else {
            const std::string a = fmt("acc%d", r0);
            b << "      for (int q = 0; q < " << E << "; ++q) " << guard << a << " = "
              << RedType(R0.op, R0.dtype).fold(a, xv) << ";\n";
        }
        b << "    }\n";
        const int g = std::min(T, 64);
        if (online) {
            b << "    for (int o = " << g / 2 << "; o >= 1; o >>= 1) rv_online_merge(om, ol, __shfl_xor(om, o, 64), __shfl_xor(ol, o, 64));\n";
            if (T > 64) {
                b << "    if ((t & 63) == 0) { red[" << slot << "][lr][lt >> 6] = om; red[" << slot + 1 << "][lr][lt >> 6] = ol; }\n";
                b << "    rv_lds_barrier();\n";
                b << "    om = red[" << slot << "][lr][0];\n    ol = red[" << slot + 1 << "][lr][0];\n";
                b << "    for (int w = 1; w < " << W << "; ++w) rv_online_merge(om, ol, red[" << slot << "][lr][w], red[" << slot + 1
                  << "][lr][w]);\n";
                slot += 2;
            }
            b << "    const float e" << r0 << " = om;\n";
            b << "    const float e" << pass[1] << " = ol;\n";
            done[r0] = done[pass[1]] = 1;
        } else {
            const RedType rt(R0.op, R0.dtype);
            b << "    " << vt(R0.dtype) << " e" << r0 << ";\n    {\n      " << rt.t << " acc = acc" << r0 << ";\n";
            b << "      acc = rv_group_" << (R0.op == RV_SUM ? "sum" : "max") << "<" << g << ">(acc);\n";
            if (T > 64) {
                b << "      if ((t & 63) == 0) red[" << slot << "][lr][lt >> 6] = acc;\n      rv_lds_barrier();\n";
                b << "      acc = (" << rt.t << ")red[" << slot << "][lr][0];\n";
                for (int w = 1; w < W; ++w)
                    b << "      acc = " << rt.fold("acc", fmt("(%s)red[%d][lr][%d]", rt.t.c_str(), slot, w)) << ";\n";
                ++slot;
            }
            if (split) {
                const int pdt = rt.isdbl ? RV_F64 : (rt.isint ? RV_I32 : RV_F32);
                const std::string P = pname(Loc{2, k.partials_region}, pdt, true);
                b << "      if (t == 0 && rv) " << P << "[r * " << lit(SP) << " + piece] = " << (rt.isint ? "(int)acc" : "acc")
                  << ";\n      e" << r0 << " = " << zero_of(R0.dtype) << ";\n    }\n";
            } else {
                b << "      e" << r0 << " = " << rt.result(R0.dtype, "acc") << ";\n    }\n";
            }
            done[r0] = 1;
        }
        emit_ready("    ");
    }
    // full-row outputs
    std::vector<int> full_roots;
    for (const Store& s_ : k.stores) {
        bool sstat = true;
        for (int d : rd)
            if (s_.v.strides[d] != 0) sstat = false;
        if (!sstat) full_roots.push_back(s_.ex);
    }
    if (!full_roots.empty()) {
        b << "    // pass: outputs\n";
        b << "    for (" << I << " c = 0; c < " << lit(NCH) << "; ++c) {\n";
        b << "      const " << I << " cb = c * " << lit(CH) << ";\n";
        emit_chunk(needed(full_roots), "      ", true);
        for (const Store& s_ : k.stores) {
            bool sstat = true;
            for (int d : rd)
                if (s_.v.strides[d] != 0) sstat = false;
            if (sstat) continue;
            std::string P = pname(s_.loc, s_.dtype, true);
            std::string val = V(s_.ex, fmt("v * %d + i", VW));
            b << "      for (int v = 0; v < " << U << "; ++v) {\n";
            b << "        const " << I << " n0 = " << nexpr("v", "0") << ";\n";
            std::vector<std::string> idx = kidx;
            bool vec = single && s_.v.strides[R] == 1 && s_.v.offset % VW == 0;
            for (int d : kd)
                if (k.domain[d] > 1 && s_.v.strides[d] % VW) vec = false;
            if (vec) {
                idx[R] = "n0";
                b << "        if (rv && n0 + " << VW << " <= " << lit(NR) << ") {\n          rv_pack<" << st(s_.dtype) << ", " << VW
                  << "> p;\n";
                b << "          for (int i = 0; i < " << VW << "; ++i) p.v[i] = " << sv(s_.dtype, val) << ";\n";
                b << "          " << vstore(s_.dtype, VW, P + " + " + addr(s_.v, idx), "p") << ";\n";
                b << "        } else\n";
            }
            b << "        for (int i = 0; i < " << VW << "; ++i) {\n          const " << I << " n = n0 + i;\n";
            red_idx(idx, "n");
            b << "          if (rv && n < " << lit(NR) << ") " << P << "[" << addr(s_.v, idx) << "] = " << sv(s_.dtype, val)
              << ";\n";
            b << "        }\n      }\n";
        }
        b << "    }\n";
    }
    for (const Store& s_ : k.stores) {
        bool sstat = true;
        for (int d : rd)
            if (s_.v.strides[d] != 0) sstat = false;
        if (!sstat) continue;
        std::string P = pname(s_.loc, s_.dtype, true);
        b << "    if (lt == 0 && rv) " << P << "[" << addr(s_.v, kidx) << "] = " << sv(s_.dtype, V(s_.ex, "0")) << ";\n";
    }
    b << "  }\n";
    return b.str();
}

// ---------------------------------------------------------------------------
// REDUCE, cells plan: one lane per output cell (lanes walk the dim that is
// stride-1 in the most buffers), the reduce dims walked in ascending order
// inside the lane, so every cell folds exactly as the serial nest does.
// ---------------------------------------------------------------------------
std::string Gen::gen_cells() {
    std::vector<int> rd, kd;
    for (int d = 0; d < rank; ++d) ((k.rdims >> d) & 1u ? rd : kd).push_back(d);
    int64_t cells = 1;
    for (int d : kd) cells *= k.domain[d];
    std::vector<int> order;  // decomposition order: other kept dims, lane dim innermost
    for (int d : kd)
        if (d != k.lane_dim) order.push_back(d);
    if (k.lane_dim >= 0) order.push_back(k.lane_dim);
    std::ostringstream b;
    b << "  for (" << I << " cell = (" << I << ")blockIdx.x * 256 + threadIdx.x; cell < " << lit(cells)
      << "; cell += (" << I << ")gridDim.x * 256) {\n";
    std::vector<std::string> idx(rank);
    {
        std::string rem = "cell";
        for (size_t j = order.size(); j-- > 0;) {
            int d = order[j];
            b << "    const " << I << " i" << d << " = " << (j ? fmt("%s %% %s", rem.c_str(), lit(k.domain[d]).c_str()) : rem)
              << ";\n";
            idx[d] = fmt("i%d", d);
            if (j) {
                b << "    const " << I << " q" << d << " = " << rem << " / " << lit(k.domain[d]) << ";\n";
                rem = fmt("q%d", d);
            }
        }
    }
    // the reduce at the root
    int root = -1;
    for (size_t e = 0; e < k.ex.size(); ++e)
        if (live[e] && (k.ex[e].op == RV_SUM || k.ex[e].op == RV_MAX)) root = (int)e;
    if (root < 0) fail(RV_E_INVALID, "internal: REDUCE kernel without a reduce");
    const Ex& R = k.ex[root];
    // invariant values (do not depend on reduce dims)
    std::vector<char> inv(k.ex.size(), 0);
    for (size_t e = 0; e < k.ex.size(); ++e) {
        const Ex& x = k.ex[e];
        if ((int)e == root) continue;
        if (x.op == RV_BUFFER) {
            const Leaf& L = k.leaves[x.leaf];
            bool s = true;
            for (int d : rd)
                if (!L.zero && (L.v.strides[d] != 0 || masked(L.v, d))) s = false;
            inv[e] = s;
        } else if (x.op == RV_CONST) {
            inv[e] = 1;
        } else {
            inv[e] = (x.a < 0 || inv[x.a]) && (x.b < 0 || inv[x.b]) && (x.c < 0 || inv[x.c]);
        }
    }
    auto emit = [&](size_t e, const std::string& ind) {
        const Ex& x = k.ex[e];
        std::string V = fmt("e%zu", e);
        if (x.op == RV_BUFFER) {
            const Leaf& L = k.leaves[x.leaf];
            if (L.zero) {
                b << ind << "const " << vt(x.dtype) << " " << V << " = " << zero_of(x.dtype) << ";\n";
                return;
            }
            std::string P = pname(L.loc, L.dtype, false);
            std::vector<int> all;
            for (int d = 0; d < rank; ++d) all.push_back(d);
            std::string mc = mask_cond(L.v, idx, all);
            b << ind << "const " << vt(x.dtype) << " " << V << " = " << (mc.empty() ? "" : "(" + mc + ") ? ")
              << ld(L.dtype, P + "[" + addr(L.v, idx) + "]") << (mc.empty() ? "" : " : " + zero_of(x.dtype)) << ";\n";
        } else if (x.op == RV_CONST) {
            b << ind << "const " << vt(x.dtype) << " " << V << " = " << const_lit(x.dtype, x.cval) << ";\n";
        } else {
            auto E = [&](int i) { return i < 0 ? std::string() : fmt("e%d", i); };
            b << ind << "const " << vt(x.dtype) << " " << V << " = " << op_code(k, x, E(x.a), E(x.b), E(x.c)) << ";\n";
        }
    };
    for (size_t e = 0; e < k.ex.size(); ++e)
        if (live[e] && inv[e] && (int)e != root) emit(e, "    ");
    const int dt = R.dtype;
    const bool sum = R.op == RV_SUM;
    std::string acc_t = dt == RV_F64 ? "double" : (is_int(dt) ? (sum ? "unsigned" : "int") : "float");
    std::string ident;
    if (sum)
        ident = dt == RV_F64 ? "0.0" : (is_int(dt) ? "0u" : "0.0f");
    else if (is_float(dt))
        ident = dt == RV_F64 ? "(-__builtin_inf())" : "(-__builtin_inff())";
    else
        ident = dt == RV_I32 ? "(-2147483647 - 1)" : (dt == RV_I16 ? "(-32768)" : "(-128)");
    b << "    " << acc_t << " acc = " << ident << ";\n";
    std::string ind = "    ";
    for (int d : rd) {
        b << ind << "for (" << I << " i" << d << " = 0; i" << d << " < " << lit(k.domain[d]) << "; ++i" << d << ") {\n";
        idx[d] = fmt("i%d", d);
        ind += "  ";
    }
    for (size_t e = 0; e < k.ex.size(); ++e)
        if (live[e] && !inv[e] && (int)e != root) emit(e, ind);
    std::string v = fmt("e%d", R.a);
    if (sum)
        b << ind << "acc = acc + " << (is_int(dt) ? "(unsigned)" + v : v) << ";\n";
    else if (is_float(dt))
        b << ind << "acc = " << (dt == RV_F64 ? "rv_maxd" : "rv_maxf") << "(acc, " << v << ");\n";
    else
        b << ind << "acc = " << v << " > acc ? " << v << " : acc;\n";
    for (size_t j = 0; j < rd.size(); ++j) {
        ind.resize(ind.size() - 2);
        b << ind << "}\n";
    }
    std::string res = is_int(dt) ? wrap_int(dt, "acc") : round_to(dt, "acc");
    b << "    const " << vt(dt) << " e" << root << " = " << res << ";\n";
    for (int d : rd) idx[d] = "";
    for (const Store& s : k.stores) {
        std::string P = pname(s.loc, s.dtype, true);
        b << "    " << P << "[" << addr(s.v, idx) << "] = " << sv(s.dtype, fmt("e%d", s.ex)) << ";\n";
    }
    b << "  }\n";
    return b.str();
}

// ---------------------------------------------------------------------------
// SPLIT, column plan: one lane per output cell (lanes walk the kept dim that
// is stride-1 in the most buffers), workgroup row blockIdx.y takes piece
// [piece * L, piece * L + L) of the reduce range (row-major over the reduced
// dims) and folds it in ascending order into its partial, written to
// partials[piece][cell] (cell = the row-major index over the kept dims).
// ---------------------------------------------------------------------------
std::string Gen::gen_split_cols() {
    std::vector<int> rd, kd;
    for (int d = 0; d < rank; ++d) ((k.rdims >> d) & 1u ? rd : kd).push_back(d);
    int64_t C = 1, N = 1;
    for (int d : kd) C *= k.domain[d];
    for (int d : rd) N *= k.domain[d];
    const int64_t P = k.split_pieces, L = (N + P - 1) / P;
    std::vector<int> order;  // other kept dims, the lane dim innermost
    for (int d : kd)
        if (d != k.lane_dim) order.push_back(d);
    if (k.lane_dim >= 0) order.push_back(k.lane_dim);
    std::ostringstream b;
    b << "  const " << I << " cell = (" << I << ")blockIdx.x * 256 + threadIdx.x;\n";
    b << "  const " << I << " piece = blockIdx.y;\n";
    b << "  if (cell >= " << lit(C) << ") return;\n";
    std::vector<std::string> idx(rank);
    {
        std::string rem = "cell";
        for (size_t j = order.size(); j-- > 0;) {
            int d = order[j];
            b << "  const " << I << " i" << d << " = " << (j ? fmt("%s %% %s", rem.c_str(), lit(k.domain[d]).c_str()) : rem)
              << ";\n";
            idx[d] = fmt("i%d", d);
            if (j) {
                b << "  const " << I << " q" << d << " = " << rem << " / " << lit(k.domain[d]) << ";\n";
                rem = fmt("q%d", d);
            }
        }
    }
    std::string lin = "0";  // row-major cell index over the kept dims
    {
        int64_t m = 1;
        for (size_t j = kd.size(); j-- > 0;) {
            lin += fmt(" + i%d * %s", kd[j], lit(m).c_str());
            m *= k.domain[kd[j]];
        }
    }
    int root = -1;
    for (size_t e = 0; e < k.ex.size(); ++e)
        if (live[e] && (k.ex[e].op == RV_SUM || k.ex[e].op == RV_MAX)) root = (int)e;
    if (root < 0) fail(RV_E_INVALID, "internal: SPLIT kernel without a reduce");
    const Ex& R = k.ex[root];
    const RedType rt(R.op, R.dtype);
    b << "  " << rt.t << " acc = " << rt.ident << ";\n";
    b << "  const " << I << " n0 = piece * " << lit(L) << ";\n";
    const bool ragged = N % L != 0;
    b << "#pragma unroll 4\n";
    b << "  for (" << I << " j = 0; j < " << lit(L) << "; ++j) {\n";
    b << "    const " << I << " n = n0 + j;\n";
    if (ragged) b << "    if (n >= " << lit(N) << ") break;\n";
    {
        std::string rem = "n";
        for (size_t j = rd.size(); j-- > 0;) {
            int d = rd[j];
            b << "    const " << I << " i" << d << " = " << (j ? fmt("%s %% %s", rem.c_str(), lit(k.domain[d]).c_str()) : rem)
              << ";\n";
            idx[d] = fmt("i%d", d);
            if (j) {
                b << "    const " << I << " r" << d << " = " << rem << " / " << lit(k.domain[d]) << ";\n";
                rem = fmt("r%d", d);
            }
        }
    }
    std::vector<char> done(k.ex.size(), 0);
    done[root] = 1;
    scalar(b, R.a, idx, "    ", "", done);
    b << "    acc = " << rt.fold("acc", fmt("s%d", R.a)) << ";\n";
    b << "  }\n";
    const int pdt = rt.isdbl ? RV_F64 : (rt.isint ? RV_I32 : RV_F32);
    const std::string Pp = pname(Loc{2, k.partials_region}, pdt, true);
    b << "  " << Pp << "[piece * " << lit(C) << " + (" << lin << ")] = " << (rt.isint ? "(int)acc" : "acc") << ";\n";
    return b.str();
}

// ---------------------------------------------------------------------------
// FOLD of a split reduce: each output cell's P partials in piece order, the
// reduce's one rounding to its dtype, then the region's elementwise tail at
// that cell and its stores. Cell-major partials: a workgroup per cell, lane t
// folds pieces t, t + 256, ... in order, then a butterfly and the 4 waves in
// order. Piece-major: 64 cells per workgroup, wave w folds the w-th quarter
// of the pieces in order for its lane's cell, then the 4 waves in order.
// Loads go 8 at a time ahead of their adds.
// ---------------------------------------------------------------------------
std::string Gen::gen_fold_cells() {
    const int64_t C = k.split_cells, P = k.split_pieces;
    const RedType rt(k.red_op, k.red_dtype);
    const int pdt = rt.isdbl ? RV_F64 : (rt.isint ? RV_I32 : RV_F32);
    const std::string Pp = pname(Loc{2, k.fold_src_region}, pdt, false);
    auto rd_part = [&](const std::string& i) {
        return rt.isint && rt.sum ? "(unsigned)" + Pp + "[" + i + "]" : Pp + "[" + i + "]";
    };
    std::ostringstream b;
    std::string ind = "  ";
    // acc folds pieces q in [q0, q1) stepping by `step`, partial index `pidx`
    auto fold_range = [&](const std::string& q0, const std::string& q1, const std::string& step,
                          const std::string& pidx) {
        b << "  for (" << I << " q = " << q0 << "; q < " << q1 << "; q += 8 * " << step << ") {\n";
        b << "    " << rt.t << " v[8];\n";
        b << "#pragma unroll\n    for (int u = 0; u < 8; ++u) {\n";
        b << "      const " << I << " qq = q + u * " << step << ";\n";
        b << "      v[u] = qq < " << q1 << " ? " << rd_part(pidx) << " : " << rt.ident << ";\n    }\n";
        b << "#pragma unroll\n    for (int u = 0; u < 8; ++u) acc = " << rt.fold("acc", "v[u]") << ";\n  }\n";
    };
    const std::string lt = rt.isdbl ? "double" : rt.isint ? (rt.sum ? "unsigned" : "int") : "float";
    if (k.split_cell_major)
        b << "  __shared__ " << lt << " wv[4][64];\n";
    else
        b << "  __shared__ " << lt << " wg[" << 256 / k.fold_cells_per_wg << "][" << k.fold_cells_per_wg << "];\n";
    b << "  const int t = threadIdx.x, lane = t & 63, w = t >> 6;\n";
    b << "  " << rt.t << " acc = " << rt.ident << ";\n";
    if (k.split_cell_major) {
        b << "  const " << I << " cell = blockIdx.x;\n";
        fold_range("(" + I + ")t", lit(P), "256", "cell * " + lit(P) + " + qq");
        if (rt.isdbl || rt.isint)
            b << "  for (int o = 32; o >= 1; o >>= 1) { const " << rt.t << " x = __shfl_xor(acc, o, 64); acc = "
              << rt.fold("acc", "x") << "; }\n";
        else
            b << "  acc = rv_group_" << (rt.sum ? "sum" : "max") << "<64>(acc);\n";
        b << "  if (lane == 0) wv[w][0] = acc;\n  __syncthreads();\n";
        b << "  if (t != 0) return;\n";
        b << "  acc = wv[0][0];\n";
        for (int j = 1; j < 4; ++j) b << "  acc = " << rt.fold("acc", fmt("wv[%d][0]", j)) << ";\n";
    } else {
        const int G = k.fold_cells_per_wg, NG = 256 / G;
        const int64_t Q = (P + NG - 1) / NG;
        b << "  const int cl = t % " << G << ", g = t / " << G << ";\n";
        b << "  const " << I << " cell = (" << I << ")blockIdx.x * " << G << " + cl;\n";
        b << "  const " << I << " cq = cell < " << lit(C) << " ? cell : " << lit(C - 1) << ";\n";
        b << "  const " << I << " pc0 = (" << I << ")g * " << lit(Q) << ", pc1 = pc0 + " << lit(Q) << " < " << lit(P)
          << " ? pc0 + " << lit(Q) << " : " << lit(P) << ";\n";
        fold_range("pc0", "pc1", "1", "qq * " + lit(C) + " + cq");
        b << "  wg[g][cl] = acc;\n  __syncthreads();\n";
        b << "  if (g != 0 || cell >= " << lit(C) << ") return;\n";
        b << "  acc = wg[0][cl];\n";
        for (int j = 1; j < NG; ++j) b << "  acc = " << rt.fold("acc", fmt("wg[%d][cl]", j)) << ";\n";
    }
    // the cell's domain indices (row-major over the output shape)
    std::vector<std::string> idx(rank);
    {
        std::string rem = "cell";
        for (int d = rank; d-- > 0;) {
            b << ind << "const " << I << " i" << d << " = " << (d ? fmt("%s %% %s", rem.c_str(), lit(k.domain[d]).c_str()) : rem)
              << ";\n";
            idx[d] = fmt("i%d", d);
            if (d) {
                b << ind << "const " << I << " q" << d << " = " << rem << " / " << lit(k.domain[d]) << ";\n";
                rem = fmt("q%d", d);
            }
        }
    }
    std::vector<char> done(k.ex.size(), 0);
    for (size_t e = 0; e < k.ex.size(); ++e)
        if (k.ex[e].op == EX_FOLD_ACC) {
            b << ind << "const " << vt(k.ex[e].dtype) << " s" << e << " = " << rt.result(k.ex[e].dtype, "acc") << ";\n";
            done[e] = 1;
        }
    for (const Store& st_ : k.stores) {
        scalar(b, st_.ex, idx, ind, "", done);
        std::string P2 = pname(st_.loc, st_.dtype, true);
        b << ind << P2 << "[" << addr(st_.v, idx) << "] = " << sv(st_.dtype, fmt("s%d", st_.ex)) << ";\n";
    }
    return b.str();
}

// ---------------------------------------------------------------------------
// SCATTER steps (limn README, "The op set", indexed; "Backends": the C
// device folds colliding adds serially, the cuda device adds atomically).
// The target already holds the base. Domain: the index's shape.
// ---------------------------------------------------------------------------
std::string Gen::gen_scatter() {
    std::ostringstream b;
    const Shape& osh = k.sc_out_shape;
    const int A = k.sc_axis, dt = k.sc_dtype;
    const int64_t CELLS = k.sc_cells, KN = k.sc_keys_n, NB = (CELLS + 2047) / 2048;
    std::vector<int64_t> os(osh.size());
    for (int64_t d = (int64_t)osh.size() - 1, st_ = 1; d >= 0; --d) {
        os[d] = st_;
        st_ *= osh[d];
    }
    std::vector<int> cd, fd;  // dims of an index cell / carried dims
    for (int d = 0; d < rank; ++d) ((k.sc_fdims >> d) & 1u ? fd : cd).push_back(d);
    auto ureg = [&](int r, bool write) {
        std::string P = pname(Loc{2, r}, RV_I32, write);
        return std::string(write ? "((unsigned*)" : "((const unsigned*)") + P + ")";
    };
    // decompose integer expression `v` over `dims` (row-major) into
    // variables <pfx><d>
    auto decompose = [&](const std::string& v, const std::vector<int>& dims, const std::string& pfx,
                         const std::string& ind) {
        std::string rem = v;
        for (size_t j = dims.size(); j-- > 0;) {
            const int d = dims[j];
            const int64_t n = k.domain[d];
            b << ind << "const long long " << pfx << d << " = " << (j ? fmt("(%s) %% %lldLL", rem.c_str(), (long long)n)
                                                                      : rem)
              << ";\n";
            if (j) {
                b << ind << "const long long " << pfx << "q" << d << " = (" << rem << ") / " << n << "LL;\n";
                rem = pfx + "q" + std::to_string(d);
            }
        }
    };
    const std::string& part = k.sc_part;
    const int cur = k.sc_pass % 2, nxt = 1 - cur;
    if (part == "hist") {
        b << "  rv_rs_hist(" << ureg(k.sc_reg_keys[cur], false) << ", " << ureg(k.sc_reg_counts, true) << ", " << CELLS
          << "LL, " << NB << "u, " << 8 * k.sc_pass << ");\n";
        return b.str();
    }
    if (part == "scan") {
        b << "  rv_rs_scan(" << ureg(k.sc_reg_counts, true) << ", " << NB << "u);\n";
        return b.str();
    }
    std::vector<int> idims;  // the dims a key walks besides the axis
    int64_t PI = 1;
    for (int d : cd)
        if (d != A) {
            idims.push_back(d);
            PI *= k.domain[d];
        }
    // the keys: target index t times the index-cell count plus the cell's
    // linear position over the index dims; an index outside the axis gets
    // the last key and its cell id flagged (bit 31) so the fold adds nothing
    auto emit_key = [&](const std::string& ind, const std::string& kout, const std::string& vout) {
        decompose("c", cd, "i", ind);
        std::vector<std::string> idx(rank, "0");
        for (int d : cd) idx[d] = fmt("i%d", d);
        std::vector<char> done(k.ex.size(), 0);
        scalar(b, k.sc_index, idx, ind, "", done);
        std::string lin = "0LL";
        int64_t m = 1;
        for (size_t j2 = idims.size(); j2-- > 0;) {
            lin += fmt(" + i%d * %lldLL", idims[j2], (long long)m);
            m *= k.domain[idims[j2]];
        }
        b << ind << "const int t = s" << k.sc_index << ";\n";
        b << ind << "const bool in = t >= 0 && t < " << osh[A] << ";\n";
        b << ind << kout << " = in ? (unsigned)((long long)t * " << PI << "LL + " << lin << ") : " << KN - 1
          << "u;\n";
        b << ind << vout << " = (unsigned)c | (in ? 0u : 0x80000000u);\n";
    };
    if (part == "move" && k.sc_fused_keys) {
        b << "  auto kf = [&](long long c, unsigned& key_, unsigned& val_) {\n";
        emit_key("    ", "key_", "val_");
        b << "  };\n";
        b << "  rv_rs_move_kv<true>(rv_rs_fn<decltype(kf)>{kf}, " << ureg(k.sc_reg_keys[nxt], true) << ", "
          << ureg(k.sc_reg_vals[nxt], true) << ", nullptr, " << CELLS << "LL, " << NB << "u, " << 8 * k.sc_pass
          << ");\n";
        return b.str();
    }
    if (part == "move") {
        const bool self = NB <= kScanInline;
        b << "  rv_rs_move<" << (self ? "true" : "false") << ">(" << ureg(k.sc_reg_keys[cur], false) << ", "
          << ureg(k.sc_reg_vals[cur], false) << ", " << ureg(k.sc_reg_keys[nxt], true) << ", "
          << ureg(k.sc_reg_vals[nxt], true) << ", "
          << (self ? std::string("nullptr") : ureg(k.sc_reg_counts, false)) << ", " << CELLS << "LL, " << NB
          << "u, " << 8 * k.sc_pass << ");\n";
        return b.str();
    }
    if (part == "bounds") {
        // a wave per 64 sorted positions: the keys between the one before
        // the chunk and the chunk's last (positions past the end count as
        // key KN) start at the first position of the chunk whose key is not
        // smaller, found by a search over the wave's 64 keys
        b << "  const unsigned* __restrict__ K = " << ureg(k.sc_reg_keys[k.sc_passes % 2], false) << ";\n";
        b << "  unsigned* __restrict__ B = " << ureg(k.sc_reg_bounds, true) << ";\n";
        b << "  const int lane = threadIdx.x & 63;\n";
        b << "  for (long long ch = ((long long)blockIdx.x * 256 + threadIdx.x) >> 6; ch <= " << CELLS / 64
          << "LL; ch += (long long)gridDim.x * 4) {\n";
        b << "    const long long p = ch * 64 + lane;\n";
        b << "    const long long key = p < " << CELLS << "LL ? (long long)K[p] : " << KN << "LL;\n";
        b << "    const long long prev = ch == 0 ? -1LL : (long long)K[ch * 64 - 1];\n";
        b << "    const long long hi = __shfl(key, 63, 64);\n";
        b << "    for (long long kb = prev + 1; kb <= hi; kb += 64) {  // uniform: every lane shuffles\n";
        b << "      const long long k = kb + lane;\n";
        b << "      int lo = 0;\n";
        b << "#pragma unroll\n";
        b << "      for (int w = 32; w >= 1; w >>= 1) {\n";
        b << "        const long long kw = __shfl(key, lo + w - 1, 64);\n";
        b << "        if (kw < k) lo += w;\n";
        b << "      }\n";
        b << "      if (k <= hi) B[k] = (unsigned)(ch * 64 + lo);\n";
        b << "    }\n";
        b << "  }\n";
        return b.str();
    }
    const std::string OUT = pname(k.sc_out, dt, true);
    if (part == "atomic") {
        std::vector<int> all;
        for (int d = 0; d < rank; ++d) all.push_back(d);
        b << "  for (long long p = (long long)blockIdx.x * 256 + threadIdx.x; p < " << numel(k.domain)
          << "LL; p += (long long)gridDim.x * 256) {\n";
        decompose("p", all, "i", "    ");
        std::vector<std::string> idx;
        for (int d = 0; d < rank; ++d) idx.push_back(fmt("i%d", d));
        std::vector<char> done(k.ex.size(), 0);
        scalar(b, k.sc_index, idx, "    ", "", done);
        scalar(b, k.sc_values, idx, "    ", "", done);
        std::string a = fmt("(long long)t * %lldLL", (long long)os[A]);
        for (int d = 0; d < rank; ++d)
            if (d != A) a += fmt(" + i%d * %lldLL", d, (long long)os[d]);
        b << "    const int t = s" << k.sc_index << ";\n";
        b << "    if (t >= 0 && t < " << osh[A] << ") rv_atomic_add(" << OUT << " + (" << a << "), s" << k.sc_values
          << ");\n";
        b << "  }\n";
        return b.str();
    }
    if (part == "keys") {
        b << "  for (long long c = (long long)blockIdx.x * 256 + threadIdx.x; c < " << CELLS
          << "LL; c += (long long)gridDim.x * 256) {\n";
        emit_key("    ", ureg(k.sc_reg_keys[0], true) + "[c]", ureg(k.sc_reg_vals[0], true) + "[c]");
        b << "  }\n";
        return b.str();
    }
    // fold: a group of TPS lanes per R consecutive target keys (every
    // output cell is one key and one carried position); a key's run of
    // sorted cells is bounds[key] .. bounds[key + 1]. For CB carried
    // positions per lane the group writes the base plus each run's values
    // in sorted (= index) order, JU cells of every key per step, so that
    // R * JU * CB loads are in flight per lane.
    const int fin = k.sc_passes % 2;
    const int64_t NF = numel(k.domain) / CELLS;
    // vector mode: CB consecutive cells of the last dim per lane (it is
    // carried and CB divides it), stored as one 16-byte (or narrower) write
    const int last = rank - 1;
    const int vcb = std::max(1, std::min(4, 16 / dtype_size(dt)));
    const bool VEC = ((k.sc_fdims >> last) & 1u) && vcb > 1 && k.domain[last] % vcb == 0;
    int TPS = 1;
    while (TPS < 256 && TPS * (VEC ? vcb : 1) < NF) TPS *= 2;
    const int SPB = 256 / TPS;
    const int CB = VEC ? vcb : (int)std::min<int64_t>(4, (NF + TPS - 1) / TPS);
    const int JU = env_int("RV_SCATTER_JU", 1);
    // values read as one vector per cell when they are a plain load that is
    // contiguous and aligned along the last dim
    const Ex& VX = k.ex[k.sc_values];
    const bool VLD = VEC && VX.op == RV_BUFFER && !k.leaves[VX.leaf].zero &&
                     !masked(k.leaves[VX.leaf].v, last) && leaf_vec_ok(k.leaves[VX.leaf], last, CB);
    int R = 4;  // plan value (lower.cpp)
    {
        const char* q = strstr(k.plan_json.c_str(), "\"keys_per_group\":");
        if (q) R = atoi(q + strlen("\"keys_per_group\":"));
    }
    b << "  const unsigned* __restrict__ VV = " << ureg(k.sc_reg_vals[fin], false) << ";\n";
    b << "  const unsigned* __restrict__ B = " << ureg(k.sc_reg_bounds, false) << ";\n";
    b << "  const int l = threadIdx.x % " << TPS << ";\n";
    b << "  for (long long k0 = ((long long)blockIdx.x * " << SPB << " + threadIdx.x / " << TPS << ") * " << R
      << "; k0 < " << KN << "LL; k0 += (long long)gridDim.x * " << SPB * R << ") {\n";
    b << "    int s[" << R << "], n[" << R << "];\n";
    b << "    long long ob[" << R << "], tk[" << R << "];\n";
    for (int d : idims) b << "    long long o" << d << "[" << R << "];\n";
    b << "    bool kv[" << R << "];\n";
    b << "    int mx = 0;\n";
    b << "#pragma unroll\n";
    b << "    for (int r = 0; r < " << R << "; ++r) {\n";
    b << "      const long long kk = k0 + r;\n";
    b << "      kv[r] = kk < " << KN << "LL;\n";
    b << "      const long long kc = kv[r] ? kk : k0;\n";
    b << "      s[r] = (int)B[kc];\n";
    b << "      n[r] = kv[r] ? (int)B[kc + 1] - s[r] : 0;\n";
    b << "      mx = n[r] > mx ? n[r] : mx;\n";
    b << "      tk[r] = kc / " << PI << "LL;\n";
    b << "      long long rem = kc % " << PI << "LL;\n";
    for (size_t j2 = idims.size(); j2-- > 0;) {
        const int d = idims[j2];
        if (j2) {
            b << "      o" << d << "[r] = rem % " << k.domain[d] << "LL;\n";
            b << "      rem = rem / " << k.domain[d] << "LL;\n";
        } else {
            b << "      o" << d << "[r] = rem;\n";
        }
    }
    std::string obs = fmt("tk[r] * %lldLL", (long long)os[A]);
    for (int d : idims) obs += fmt(" + o%d[r] * %lldLL", d, (long long)os[d]);
    b << "      ob[r] = " << obs << ";\n";
    b << "    }\n";
    b << "    for (long long f0 = (long long)l" << (VEC ? fmt(" * %d", CB) : std::string()) << "; f0 < " << NF
      << "LL; f0 += " << (int64_t)TPS * CB << "LL) {\n";
    b << "      " << vt(dt) << " acc[" << R << "][" << CB << "];\n";
    b << "      long long fo[" << CB << "];\n";
    for (int d : fd) b << "      long long fc" << d << "[" << CB << "];\n";
    b << "#pragma unroll\n";
    b << "      for (int cb = 0; cb < " << CB << "; ++cb) {\n";
    b << "        const long long f = f0 + (long long)cb" << (VEC ? std::string() : fmt(" * %d", TPS)) << ";\n";
    b << "        const long long fcl = f < " << NF << "LL ? f : " << NF - 1 << "LL;\n";
    decompose("fcl", fd, "fi", "        ");
    std::string fo = "0LL";
    for (int d : fd) {
        b << "        fc" << d << "[cb] = fi" << d << ";\n";
        fo += fmt(" + fi%d * %lldLL", d, (long long)os[d]);
    }
    b << "        fo[cb] = " << fo << ";\n";
    b << "#pragma unroll\n";
    b << "        for (int r = 0; r < " << R << "; ++r) {\n";
    {
        std::vector<std::string> bidx(rank);
        bidx[A] = "tk[r]";
        for (int d : idims) bidx[d] = fmt("o%d[r]", d);
        for (int d : fd) bidx[d] = fmt("fi%d", d);
        std::vector<char> done(k.ex.size(), 0);
        scalar(b, k.sc_base, bidx, "          ", "b", done);
        b << "          acc[r][cb] = s" << k.sc_base << "b;\n";
    }
    b << "        }\n";
    b << "      }\n";
    b << "      for (int j0 = 0; j0 < mx; j0 += " << JU << ") {\n";
    b << "        unsigned cj[" << R << "][" << JU << "];\n";
    b << "        bool add[" << R << "][" << JU << "];\n";
    b << "#pragma unroll\n";
    b << "        for (int r = 0; r < " << R << "; ++r)\n";
    b << "#pragma unroll\n";
    b << "          for (int u = 0; u < " << JU << "; ++u) {\n";
    b << "            const unsigned c = j0 + u < n[r] ? VV[s[r] + j0 + u] : 0x80000000u;\n";
    b << "            add[r][u] = !(c & 0x80000000u);\n";
    b << "            cj[r][u] = min(c & 0x7fffffffu, " << CELLS - 1 << "u);\n";
    b << "          }\n";
    b << "        " << vt(dt) << " vv[" << R << "][" << JU << "][" << CB << "];\n";
    b << "#pragma unroll\n";
    b << "        for (int r = 0; r < " << R << "; ++r)\n";
    b << "#pragma unroll\n";
    b << "        for (int u = 0; u < " << JU << "; ++u) {\n";
    decompose("(long long)cj[r][u]", cd, "i", "          ");
    if (VLD) {
        const Leaf& L = k.leaves[VX.leaf];
        std::vector<std::string> idx(rank);
        for (int d : cd) idx[d] = fmt("i%d", d);
        for (int d : fd) idx[d] = fmt("fc%d[0]", d);
        std::vector<int> all;
        for (int d = 0; d < rank; ++d) all.push_back(d);
        const std::string mc = mask_cond(L.v, idx, all);
        b << "          if (add[r][u]" << (mc.empty() ? "" : " && " + mc) << ") {\n";
        b << "            const rv_pack<" << st(dt) << ", " << CB << "> v = "
          << vload(L, CB, pname(L.loc, L.dtype, false) + " + " + addr(L.v, idx)) << ";\n";
        b << "#pragma unroll\n";
        b << "            for (int cb = 0; cb < " << CB << "; ++cb) vv[r][u][cb] = " << ld(dt, "v.v[cb]") << ";\n";
        b << "          } else {\n";
        b << "#pragma unroll\n";
        b << "            for (int cb = 0; cb < " << CB << "; ++cb) vv[r][u][cb] = " << zero_of(dt) << ";\n";
        b << "          }\n";
    } else {
        b << "#pragma unroll\n";
        b << "          for (int cb = 0; cb < " << CB << "; ++cb) {\n";
        std::vector<std::string> idx(rank);
        for (int d : cd) idx[d] = fmt("i%d", d);
        for (int d : fd) idx[d] = fmt("fc%d[cb]", d);
        std::vector<char> done(k.ex.size(), 0);
        b << "            if (add[r][u]) {\n";
        scalar(b, k.sc_values, idx, "              ", "", done);
        b << "              vv[r][u][cb] = s" << k.sc_values << ";\n";
        b << "            } else {\n";
        b << "              vv[r][u][cb] = " << zero_of(dt) << ";\n";
        b << "            }\n";
        b << "          }\n";
    }
    b << "        }\n";
    Ex add;
    add.op = RV_ADD;
    add.dtype = dt;
    b << "#pragma unroll\n";
    b << "        for (int r = 0; r < " << R << "; ++r)\n";
    b << "#pragma unroll\n";
    b << "          for (int u = 0; u < " << JU << "; ++u)\n";
    b << "#pragma unroll\n";
    b << "            for (int cb = 0; cb < " << CB << "; ++cb)\n";
    b << "              if (add[r][u]) acc[r][cb] = " << op_code(k, add, "acc[r][cb]", "vv[r][u][cb]", "") << ";\n";
    b << "      }\n";
    b << "#pragma unroll\n";
    b << "      for (int r = 0; r < " << R << "; ++r)\n";
    if (VEC) {  // CB divides NF: every lane's CB cells are in range together
        b << "        if (kv[r]) {\n";
        b << "          rv_pack<" << st(dt) << ", " << CB << "> v;\n";
        b << "#pragma unroll\n";
        b << "          for (int cb = 0; cb < " << CB << "; ++cb) v.v[cb] = " << sv(dt, "acc[r][cb]") << ";\n";
        b << "          " << vstore(dt, CB, OUT + " + ob[r] + fo[0]", "v") << ";\n";
        b << "        }\n";
    } else {
        b << "#pragma unroll\n";
        b << "        for (int cb = 0; cb < " << CB << "; ++cb)\n";
        b << "          if (kv[r] && f0 + (long long)cb * " << TPS << " < " << NF << "LL) " << OUT
          << "[ob[r] + fo[cb]] = " << sv(dt, "acc[r][cb]") << ";\n";
    }
    b << "    }\n";
    b << "  }\n";
    return b.str();
}

// ATTN: the fused attention forward skeleton (kernels/rv_device.hpp) with
// the head width, causal flag, output dtype and the base-2 score scale
// baked in.
std::string Gen::gen_attn() {
    const int64_t Tq = k.domain[1], D = k.domain[2];
    const int64_t Tk = k.leaves[1].v.shape[1];
    std::string q, kp, v;
    if (!k.attn_merge) {
        q = pname(k.leaves[0].loc, RV_BF16, false);
        kp = pname(k.leaves[1].loc, RV_BF16, false);
        v = pname(k.leaves[2].loc, RV_BF16, false);
    }
    std::string o = "nullptr", l = "nullptr";
    int odt = RV_F32;
    int no = 0, nl = 0;
    for (const Store& st_ : k.stores) {
        if (st_.out_index == 0) {
            o = pname(st_.loc, st_.dtype, true);
            odt = st_.dtype;
            ++no;
        } else {
            l = pname(st_.loc, RV_F32, true);
            ++nl;
        }
    }
    if (no > 1 || nl > 1) fail(RV_E_UNSUPPORTED_LAYOUT, "sdpa_fwd: one output requested twice");
    const float sl2 = (float)(k.attn_scale * 1.4426950408889634);  // scale * log2(e)
    const std::string causal = k.attn_causal ? "true" : "false", obf = odt == RV_BF16 ? "true" : "false";
    std::ostringstream pre, b;
    if (k.attn_merge) {
        const std::string op = pname(Loc{2, k.attn_reg_o}, RV_F32, false);
        const std::string ml = pname(Loc{2, k.attn_reg_ml}, RV_F32, false);
        b << "  rv_attn_merge_chunks<" << D << ", " << causal << ", " << obf << ">(" << o << ", " << l << ", " << op
          << ", " << ml << ", " << Tq << ", " << Tk << ", " << k.attn_chunk << ", " << k.attn_cmax << ");\n";
        return "@@BODY@@" + b.str();
    }
    b << "  rv_attn_fwd_bf16<" << D << ", " << causal << ", " << obf << ", " << k.attn_stages << ">(" << q << ", "
      << kp << ", " << v << ", " << o << ", " << l << ", " << Tq << ", " << Tk << ", " << fmt("%a", sl2) << "f";
    if (k.attn_chunk > 0) {
        // the (query block, key chunk) of every workgroup, longest blocks first
        pre << "__constant__ unsigned " << k.name << "_map[" << k.attn_map.size() << "] = {";
        for (size_t i = 0; i < k.attn_map.size(); ++i) pre << (i ? (i % 16 ? ", " : ",\n  ") : "") << k.attn_map[i] << "u";
        pre << "};\n";
        const std::string op = pname(Loc{2, k.attn_reg_o}, RV_F32, true);
        const std::string ml = pname(Loc{2, k.attn_reg_ml}, RV_F32, true);
        b << ", " << k.name << "_map, " << k.attn_chunk << ", " << op << ", " << ml << ", " << k.attn_cmax;
    }
    b << ");\n";
    return pre.str() + "@@BODY@@" + b.str();
}

std::string Gen::gen_fold() {
    const Ex& R = k.ex[0];
    std::string src = pname(Loc{2, k.fold_src_region}, RV_F32, false);
    std::ostringstream b;
    b << "  const float s = rv_fold_sum(" << src << ", " << k.fold_count << "LL);\n";
    for (const Store& s : k.stores) {
        std::string P = pname(s.loc, s.dtype, true);
        b << "  if (threadIdx.x == 0) " << P << "[" << s.v.offset << "] = " << sv(s.dtype, round_to(R.dtype, "s")) << ";\n";
    }
    return b.str();
}

// ---------------------------------------------------------------------------
// MFMA: the hand-written contraction skeleton plus a generated epilogue
// functor that evaluates the graph's elementwise tail on y at (m, n).
// ---------------------------------------------------------------------------
std::string Gen::gen_gemm() {
    const Leaf& A = k.leaves[k.mfma_a];
    const Leaf& B = k.leaves[k.mfma_b];
    const bool kn = B.v.strides[1] == 1;
    const int64_t Mt = k.domain[0], Nt = k.domain[1];
    const int64_t M = k.mfma_ext[0], N = k.mfma_ext[1], K = k.mfma_ext[2];
    const bool ragged = M % 256 || N % 256 || M != Mt || N != Nt;
    const int64_t lda = A.v.strides[0];
    const int64_t ldb = kn ? B.v.strides[2] : B.v.strides[1];
    const int64_t plane = (Mt * Nt + 63) / 64 * 64;
    const Kernel::GemmSched& g = k.gemm;
    if (k.mfma_split > 1 && !k.mfma_slices) {
        // slice s = blockIdx % S of the k-range: its operand offsets, depth
        // and plane
        const int S = k.mfma_split;
        const int64_t Ks = K / S;
        std::string pa = pname(A.loc, RV_BF16, false);
        std::string pb = pname(B.loc, RV_BF16, false);
        std::string pw = pname(Loc{2, k.slices_region}, RV_F32, true);
        std::ostringstream b;
        b << "  const long long s_ = (long long)(blockIdx.x % " << S << "u);\n";
        b << "  const rv_slice_epi epi{" << pw << " + s_ * " << plane << "LL, " << Nt << "};\n";
        b << "  rv_gemm_w6_bf16<" << (kn ? "true" : "false") << ", 0, rv_slice_epi, " << g.pin << ", "
          << (ragged ? "true" : "false") << ", " << g.pe << ", " << g.po << ", " << S << ">(" << pa << ", " << pb
          << ", " << A.v.offset << "LL + s_ * " << Ks << "LL, " << lda << "LL, " << B.v.offset << "LL + s_ * "
          << Ks * (kn ? ldb : 1) << "LL, " << ldb << "LL, " << M << ", " << N << ", " << Ks << ", epi, nullptr, " << Mt
          << ", " << Nt << ");\n";
        return "@@BODY@@" + b.str();
    }
    std::string pa = k.mfma_slices ? std::string() : pname(A.loc, RV_BF16, false);
    std::string pb = k.mfma_slices ? std::string() : pname(B.loc, RV_BF16, false);
    std::ostringstream f;  // functor body
    std::string sname = k.name + "_epi";
    std::vector<std::string> idx = {"m", "n", ""};
    std::ostringstream body;
    int final_ex = k.stores[0].ex;
    for (size_t e = 0; e < k.ex.size(); ++e) {
        if (!live[e]) continue;
        const Ex& x = k.ex[e];
        std::string V = fmt("e%zu", e);
        if (x.op == EX_MFMA_ACC) {
            body << "    const float " << V << " = acc;\n";
        } else if (x.op == RV_BUFFER) {
            const Leaf& L = k.leaves[x.leaf];
            if (L.zero) {
                body << "    const " << vt(x.dtype) << " " << V << " = " << zero_of(x.dtype) << ";\n";
                continue;
            }
            std::string P = pname(L.loc, L.dtype, false);
            std::string mc = mask_cond(L.v, idx, {0, 1});
            body << "    const " << vt(x.dtype) << " " << V << " = " << (mc.empty() ? "" : "(" + mc + ") ? ")
                 << ld(L.dtype, "P" + P + "[" + addr(L.v, idx) + "]") << (mc.empty() ? "" : " : " + zero_of(x.dtype))
                 << ";\n";
        } else if (x.op == RV_CONST) {
            body << "    const " << vt(x.dtype) << " " << V << " = " << const_lit(x.dtype, x.cval) << ";\n";
        } else {
            auto E = [&](int i) { return i < 0 ? std::string() : fmt("e%d", i); };
            body << "    const " << vt(x.dtype) << " " << V << " = " << op_code(k, x, E(x.a), E(x.b), E(x.c)) << ";\n";
        }
    }
    std::ostringstream stores;
    if (!k.mfma_partial)
        for (const Store& s : k.stores) {
            std::string P = pname(s.loc, s.dtype, true);
            stores << "    P" << P << "[" << addr(s.v, idx) << "] = " << sv(s.dtype, "v") << ";\n";
        }
    std::string partials;
    if (k.mfma_partial) partials = pname(Loc{2, k.partials_region}, RV_F32, true);
    // functor holds every parameter pointer (prefixed P)
    std::string sig = signature();
    f << "struct " << sname << " {\n";
    for (size_t i = 0; i < params.size(); ++i)
        f << "  " << (written[i] ? "" : "const ") << st(param_dtype[i]) << "* __restrict__ Pp" << i << ";\n";
    f << "  __device__ __forceinline__ float operator()(float acc, int m, int n) const {\n" << body.str();
    f << "    return (float)(e" << final_ex << ");\n  }\n";
    f << "  __device__ __forceinline__ void store(int m, int n, float v) const {\n" << stores.str() << "  }\n};\n";
    std::ostringstream b;
    b << "  const " << sname << " epi{";
    for (size_t i = 0; i < params.size(); ++i) b << (i ? ", " : "") << "p" << i;
    b << "};\n";
    if (k.mfma_slices) {
        std::string pw = pname(Loc{2, k.slices_region}, RV_F32, false);
        b << "  rv_gemm_slices<" << (k.mfma_partial ? 1 : 0) << ", " << sname << ">(" << pw << ", " << k.mfma_split
          << ", " << plane << "LL, " << Mt << ", " << Nt << ", epi, "
          << (k.mfma_partial ? partials : std::string("nullptr")) << ");\n";
        return f.str() + "@@BODY@@" + b.str();
    }
    b << "  rv_gemm_w6_bf16<" << (kn ? "true" : "false") << ", " << (k.mfma_partial ? 1 : 0) << ", " << sname << ", "
      << g.pin << ", " << (ragged ? "true" : "false") << ", " << g.pe << ", " << g.po << ">(" << pa << ", " << pb << ", ";
    b
      << A.v.offset << "LL, " << lda << "LL, " << B.v.offset << "LL, " << ldb << "LL, " << M << ", " << N << ", " << K
      << ", epi, " << (k.mfma_partial ? partials : std::string("nullptr")) << ", " << Mt << ", " << Nt << ");\n";
    return f.str() + "@@BODY@@" + b.str();
}

std::string Gen::gen() {
    std::string body;
    std::string pre;
    if (k.plan == "empty") return "";
    switch (k.cls) {
        case KClass::EW: body = k.plan == "tiled2d" ? gen_tiled() : gen_rowmajor(); break;
        case KClass::ROW: body = k.plan == "row_stream" ? gen_row_stream() : gen_row(); break;
        case KClass::REDUCE: body = gen_cells(); break;
        case KClass::FOLD: body = k.plan == "fold_cells" ? gen_fold_cells() : gen_fold(); break;
        case KClass::SPLIT: body = k.plan == "split_row" ? gen_row_stream() : gen_split_cols(); break;
        case KClass::ATTN: {
            std::string s = gen_attn();
            size_t at = s.find("@@BODY@@");
            pre = s.substr(0, at);
            body = s.substr(at + 8);
            break;
        }
        case KClass::SCATTER: body = gen_scatter(); break;
        case KClass::MFMA: {
            std::string s = gen_gemm();
            size_t at = s.find("@@BODY@@");
            pre = s.substr(0, at);
            body = s.substr(at + 8);
            break;
        }
    }
    return pre + header() + " {\n" + body + "}\n";
}

}  // namespace

std::string codegen(const Program& p) {
    std::string s = "// generated by reduce_view for gfx950\n";
    s += kDeviceHeader;
    s += "\n";
    for (const Kernel& k : p.kernels) {
        Gen g(p, k);
        s += "\n" + g.gen();
    }
    return s;
}

// Parameter list of a kernel, in the order its generated signature uses.
std::vector<Loc> kernel_param_locs(const Program& p, const Kernel& k) {
    Gen g(p, k);
    g.gen();
    return g.params;
}

}  // namespace rv
