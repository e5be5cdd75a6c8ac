// The C ABI (include/rv.h): every entry point turns internal errors into a
// typed status plus a thread-local message naming the broken contract (Tiki
// README, "Compile model code"); nothing throws across the boundary.
#include <cstring>
#include <memory>

#include "graph.hpp"

struct rv_program {
    rv::Program p;
};

namespace {

thread_local std::string g_err;

rv_status ok() {
    g_err.clear();
    return RV_OK;
}

template <class F>
rv_status guard(F&& f) {
    try {
        f();
        return ok();
    } catch (const rv::Error& e) {
        g_err = e.msg;
        return e.status;
    } catch (const std::bad_alloc&) {
        g_err = "host out of memory";
        return RV_E_INVALID;
    } catch (const std::exception& e) {
        g_err = std::string("internal error: ") + e.what();
        return RV_E_INVALID;
    } catch (...) {
        g_err = "internal error";
        return RV_E_INVALID;
    }
}

rv_status copy_out(const std::string& s, char* out, size_t cap, size_t* needed) {
    if (needed) *needed = s.size() + 1;
    if (out && cap) {
        size_t n = std::min(cap - 1, s.size());
        memcpy(out, s.data(), n);
        out[n] = '\0';
    }
    return ok();
}

rv::Shape shape_of(const int64_t* s, int32_t n) {
    if (n < 0 || n > RV_MAX_DIMS) rv::fail(RV_E_INVALID, "rank outside [0, 8]");
    if (n && !s) rv::fail(RV_E_INVALID, "NULL shape");
    return rv::Shape(s, s + n);
}

}  // namespace

extern "C" {

rv_status rv_init(int device) { return guard([&] { rv::device_check(device); }); }

rv_status rv_compile(const rv_node* nodes, int32_t n, const int32_t* outputs, int32_t nout, rv_program** out) {
    return guard([&] {
        if (!out) rv::fail(RV_E_INVALID, "NULL output handle");
        *out = nullptr;
        std::unique_ptr<rv_program> prog(new rv_program);
        rv::Program& p = prog->p;
        p.g = rv::intake(nodes, n, outputs, nout);
        rv::schedule(p);
        rv::lower(p);
        p.source = rv::codegen(p);
        p.kparams.clear();
        for (const auto& k : p.kernels) p.kparams.push_back(rv::kernel_param_locs(p, k));
        rv::compile_code(p);
        *out = prog.release();
    });
}

rv_status rv_node_shape(const rv_node* nodes, int32_t n, int32_t i, rv_view* shape, int32_t* dtype) {
    return guard([&] {
        if (!nodes || i < 0 || i >= n) rv::fail(RV_E_INVALID, "node index out of range");
        rv::Graph g = rv::intake(nodes, i + 1, &i, 1);
        if (shape) *shape = rv::view_contiguous(g.nodes[i].shape);
        if (dtype) *dtype = g.nodes[i].dtype;
    });
}

rv_status rv_program_io(const rv_program* prog, int32_t* n_inputs, int32_t* n_outputs) {
    return guard([&] {
        if (!prog) rv::fail(RV_E_INVALID, "NULL program");
        if (n_inputs) *n_inputs = prog->p.g.n_inputs;
        if (n_outputs) *n_outputs = (int32_t)prog->p.outputs.size();
    });
}

rv_status rv_output_desc(const rv_program* prog, int32_t i, rv_view* shape, int32_t* dtype) {
    return guard([&] {
        if (!prog) rv::fail(RV_E_INVALID, "NULL program");
        if (i < 0 || i >= (int32_t)prog->p.outputs.size()) rv::fail(RV_E_INVALID, "output index out of range");
        if (shape) *shape = rv::view_contiguous(prog->p.outputs[i].shape);
        if (dtype) *dtype = prog->p.outputs[i].dtype;
    });
}

rv_status rv_workspace_size(const rv_program* prog, size_t* bytes) {
    return guard([&] {
        if (!prog || !bytes) rv::fail(RV_E_INVALID, "NULL argument");
        *bytes = prog->p.ws_bytes;
    });
}

rv_status rv_launch(const rv_program* prog, const rv_buffer* bufs, int32_t nbufs, void* workspace, size_t ws_bytes,
                    void* stream) {
    return guard([&] {
        if (!prog) rv::fail(RV_E_INVALID, "NULL program");
        rv::launch(const_cast<rv::Program&>(prog->p), bufs, nbufs, workspace, ws_bytes, stream);
    });
}

rv_status rv_launch_noalloc(const rv_program* prog, const rv_buffer* bufs, int32_t nbufs, void* stream) {
    return guard([&] {
        if (!prog) rv::fail(RV_E_INVALID, "NULL program");
        rv::launch_noalloc(const_cast<rv::Program&>(prog->p), bufs, nbufs, stream);
    });
}

rv_status rv_describe(const rv_program* prog, char* out, size_t cap, size_t* needed) {
    std::string s;
    rv_status st = guard([&] {
        if (!prog) rv::fail(RV_E_INVALID, "NULL program");
        s = rv::describe(prog->p);
    });
    return st != RV_OK ? st : copy_out(s, out, cap, needed);
}

rv_status rv_source(const rv_program* prog, char* out, size_t cap, size_t* needed) {
    if (!prog) {
        g_err = "NULL program";
        return RV_E_INVALID;
    }
    return copy_out(prog->p.source, out, cap, needed);
}

void rv_program_free(rv_program* prog) { delete prog; }

const char* rv_last_error(void) { return g_err.c_str(); }

rv_status rv_view_contiguous(const int64_t* shape, int32_t ndim, rv_view* out) {
    return guard([&] {
        if (!out) rv::fail(RV_E_INVALID, "NULL output view");
        *out = rv::view_contiguous(shape_of(shape, ndim));
    });
}

rv_status rv_view_reshape(const rv_view* in, const int64_t* shape, int32_t ndim, rv_view* out) {
    return guard([&] {
        if (!in || !out) rv::fail(RV_E_INVALID, "NULL view");
        *out = rv::view_reshape(*in, shape_of(shape, ndim));
    });
}

rv_status rv_view_permute(const rv_view* in, const int32_t* perm, rv_view* out) {
    return guard([&] {
        if (!in || !out || (!perm && in->ndim)) rv::fail(RV_E_INVALID, "NULL argument");
        std::vector<int> pv(perm, perm + in->ndim);
        *out = rv::view_permute(*in, pv);
    });
}

rv_status rv_view_expand(const rv_view* in, const int64_t* shape, rv_view* out) {
    return guard([&] {
        if (!in || !out) rv::fail(RV_E_INVALID, "NULL view");
        *out = rv::view_expand(*in, shape_of(shape, in->ndim));
    });
}

rv_status rv_view_pad(const rv_view* in, const int64_t* before, const int64_t* after, rv_view* out) {
    return guard([&] {
        if (!in || !out) rv::fail(RV_E_INVALID, "NULL view");
        *out = rv::view_pad(*in, shape_of(before, in->ndim), shape_of(after, in->ndim));
    });
}

rv_status rv_view_shrink(const rv_view* in, const int64_t* lo, const int64_t* hi, rv_view* out) {
    return guard([&] {
        if (!in || !out) rv::fail(RV_E_INVALID, "NULL view");
        *out = rv::view_shrink(*in, shape_of(lo, in->ndim), shape_of(hi, in->ndim));
    });
}

}  // extern "C"
