// Runtime: compiles a program's generated HIP source for gfx950 with the HIP
// runtime compiler, caches code objects by a hash of everything that decides
// the bytes (source, options, compiler version, target; Tiki README,
// "Milestones", gate 4), loads them per device and launches kernels on the
// caller's stream (Tiki README, "What works today": caller-owned buffers and
// stream). The library never allocates device memory and never synchronises.
#include <hip/hip_runtime.h>
#include <hip/hiprtc.h>
#include <sys/stat.h>
#include <unistd.h>

#include <cstdlib>
#include <cstring>
#include <fstream>
#include <map>
#include <mutex>
#include <sstream>

#include "graph.hpp"

namespace rv {

static const char* const kOptions[] = {
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
    // packed FP32 instructions stay off: hipcc forms them from plain float code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
};

static uint64_t fnv1a(const std::string& s, uint64_t h) {
    for (unsigned char c : s) {
        h ^= c;
        h *= 1099511628211ull;
    }
    return h;
}

static std::string compiler_id() {
    int v = 0;
    hiprtcVersion(&v, nullptr);
    int major = 0, minor = 0;
    hiprtcVersion(&major, &minor);
    return fmt("hiprtc-%d.%d", major, minor);
}

static std::mutex g_cache_mu;
static std::map<std::string, std::vector<char>> g_cache;

static std::string cache_dir() {
    const char* d = getenv("RV_CACHE_DIR");
    if (d && *d) return d;
    const char* h = getenv("HOME");
    if (!h || !*h) return "";
    return std::string(h) + "/.cache/reduce_view_amd";
}

static bool read_file(const std::string& path, std::vector<char>* out) {
    std::ifstream f(path, std::ios::binary);
    if (!f) return false;
    std::ostringstream ss;
    ss << f.rdbuf();
    std::string s = ss.str();
    out->assign(s.begin(), s.end());
    return !out->empty();
}

static void write_file_atomic(const std::string& dir, const std::string& name, const std::vector<char>& data) {
    if (dir.empty()) return;
    std::string cur;
    for (size_t i = 0; i <= dir.size(); ++i) {
        if (i == dir.size() || dir[i] == '/') {
            if (!cur.empty()) mkdir(cur.c_str(), 0755);
        }
        if (i < dir.size()) cur += dir[i];
    }
    std::string tmp = dir + "/" + name + fmt(".tmp%d", (int)getpid());
    {
        std::ofstream f(tmp, std::ios::binary);
        if (!f) return;
        f.write(data.data(), (std::streamsize)data.size());
        if (!f) return;
    }
    rename(tmp.c_str(), (dir + "/" + name).c_str());
}

void compile_code(Program& p) {
    std::string opts;
    for (const char* o : kOptions) opts += std::string(o) + " ";
    p.options = opts;
    std::string ident = p.source + "\n//" + opts + compiler_id() + " gfx950";
    p.key = fmt("%016llx%016llx", (unsigned long long)fnv1a(ident, 1469598103934665603ull),
                (unsigned long long)fnv1a(ident, 0x84222325cbf29ce4ull));
    // RV_DEBUG_BAD_SOURCE=1 appends a line the compiler rejects, bypassing
    // every cache, so the RV_E_COMPILE path can be exercised on purpose.
    const char* bad = getenv("RV_DEBUG_BAD_SOURCE");
    const bool inject = bad && *bad && std::string(bad) != "0";
    if (!inject) {
        std::lock_guard<std::mutex> lk(g_cache_mu);
        auto it = g_cache.find(p.key);
        if (it != g_cache.end()) {
            p.code = it->second;
            return;
        }
    }
    const std::string dir = cache_dir();
    if (!inject && !dir.empty()) {
        std::vector<char> code, src;
        if (read_file(dir + "/" + p.key + ".co", &code) && read_file(dir + "/" + p.key + ".hip", &src) &&
            std::string(src.begin(), src.end()) == ident) {
            p.code = code;
            std::lock_guard<std::mutex> lk(g_cache_mu);
            g_cache[p.key] = code;
            return;
        }
    }
    std::string src = inject ? p.source + "\n#error injected compile failure\n" : p.source;
    hiprtcProgram prog;
    if (hiprtcCreateProgram(&prog, src.c_str(), "rv_program.hip", 0, nullptr, nullptr) != HIPRTC_SUCCESS)
        fail(RV_E_COMPILE, "hiprtcCreateProgram failed");
    const int nopt = (int)(sizeof kOptions / sizeof kOptions[0]);
    hiprtcResult r = hiprtcCompileProgram(prog, nopt, kOptions);
    size_t log_size = 0;
    hiprtcGetProgramLogSize(prog, &log_size);
    std::string log(log_size + 1, '\0');
    if (log_size) hiprtcGetProgramLog(prog, &log[0]);
    if (r != HIPRTC_SUCCESS) {
        hiprtcDestroyProgram(&prog);
        if (log.size() > 3000) log = log.substr(0, 3000) + "...";
        fail(RV_E_COMPILE, std::string("the HIP runtime compiler rejected the generated kernels: ") + log.c_str());
    }
    size_t size = 0;
    hiprtcGetCodeSize(prog, &size);
    std::vector<char> code(size);
    hiprtcGetCode(prog, code.data());
    hiprtcDestroyProgram(&prog);
    p.code = code;
    if (inject) return;
    {
        std::lock_guard<std::mutex> lk(g_cache_mu);
        g_cache[p.key] = code;
    }
    write_file_atomic(dir, p.key + ".co", code);
    write_file_atomic(dir, p.key + ".hip", std::vector<char>(ident.begin(), ident.end()));
}

void device_check(int device) {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n == 0) fail(RV_E_DEVICE, "no HIP device is visible");
    if (device < 0 || device >= n) fail(RV_E_DEVICE, fmt("device %d does not exist (%d visible)", device, n));
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) fail(RV_E_DEVICE, "hipGetDeviceProperties failed");
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        fail(RV_E_DEVICE, fmt("device %d is %s; this library is built for gfx950 (MI355X) only", device,
                              prop.gcnArchName));
}

static void ensure_loaded(Program& p, int dev, std::vector<void*>** fns) {
    std::lock_guard<std::mutex> lk(p.mu);
    auto it = p.functions.find(dev);
    if (it != p.functions.end()) {
        *fns = &it->second;
        return;
    }
    static std::mutex checked_mu;
    static std::map<int, bool> checked;
    {
        std::lock_guard<std::mutex> lk2(checked_mu);
        if (!checked[dev]) {
            device_check(dev);
            checked[dev] = true;
        }
    }
    hipModule_t mod;
    hipError_t e = hipModuleLoadData(&mod, p.code.data());
    if (e != hipSuccess) fail(RV_E_LAUNCH, fmt("hipModuleLoadData: %s", hipGetErrorString(e)));
    std::vector<void*> f(p.kernels.size(), nullptr);
    for (size_t i = 0; i < p.kernels.size(); ++i) {
        if (p.kernels[i].plan == "empty") continue;
        hipFunction_t fn;
        e = hipModuleGetFunction(&fn, mod, p.kernels[i].name.c_str());
        if (e != hipSuccess) fail(RV_E_LAUNCH, fmt("hipModuleGetFunction(%s): %s", p.kernels[i].name.c_str(),
                                                   hipGetErrorString(e)));
        f[i] = (void*)fn;
    }
    p.modules[dev] = (void*)mod;
    p.functions[dev] = f;
    *fns = &p.functions[dev];
}

bool loaded_on(Program& p, int dev) {
    std::lock_guard<std::mutex> lk(p.mu);
    return p.functions.find(dev) != p.functions.end();
}

void launch(Program& p, const rv_buffer* bufs, int32_t nbufs, void* ws, size_t ws_bytes, void* stream) {
    const int nin = p.g.n_inputs, nout = (int)p.outputs.size();
    if (nbufs != nin + nout || (!bufs && nbufs))
        fail(RV_E_INVALID, fmt("expected %d buffers (%d inputs + %d outputs), got %d", nin + nout, nin, nout, nbufs));
    struct Range {
        uintptr_t lo, hi;
    };
    std::vector<Range> in_ranges;
    for (int i = 0; i < nin; ++i) {
        const rv_buffer& b = bufs[i];
        if (p.input_dtype[i] < 0) continue;  // slot unused by the graph
        if (b.dtype != p.input_dtype[i])
            fail(RV_E_DTYPE, fmt("input %d is %s, the graph declares %s", i, dtype_name(b.dtype),
                                 dtype_name(p.input_dtype[i])));
        if (b.nelems < p.input_nelems[i])
            fail(RV_E_INVALID, fmt("input %d holds %lld elements, the graph reads %lld", i, (long long)b.nelems,
                                   (long long)p.input_nelems[i]));
        if (p.input_nelems[i] > 0 && !b.ptr) fail(RV_E_INVALID, fmt("input %d is NULL", i));
        in_ranges.push_back({(uintptr_t)b.ptr, (uintptr_t)b.ptr + (uintptr_t)b.nelems * dtype_size(b.dtype)});
    }
    for (int o = 0; o < nout; ++o) {
        const rv_buffer& b = bufs[nin + o];
        const OutputInfo& oi = p.outputs[o];
        if (b.dtype != oi.dtype)
            fail(RV_E_DTYPE, fmt("output %d is %s, the graph produces %s", o, dtype_name(b.dtype), dtype_name(oi.dtype)));
        if (b.nelems < numel(oi.shape))
            fail(RV_E_INVALID, fmt("output %d holds %lld elements, needs %lld", o, (long long)b.nelems,
                                   (long long)numel(oi.shape)));
        if (numel(oi.shape) > 0 && !b.ptr) fail(RV_E_INVALID, fmt("output %d is NULL", o));
        uintptr_t lo = (uintptr_t)b.ptr, hi = lo + (uintptr_t)numel(oi.shape) * dtype_size(oi.dtype);
        for (auto& r : in_ranges)
            if (lo < r.hi && r.lo < hi && hi > lo) fail(RV_E_INVALID, fmt("output %d overlaps an input", o));
    }
    if (p.ws_bytes > 0) {
        if (!ws) fail(RV_E_WORKSPACE, fmt("the program needs %zu bytes of workspace", p.ws_bytes));
        if (ws_bytes < p.ws_bytes)
            fail(RV_E_WORKSPACE, fmt("workspace of %zu bytes is smaller than the %zu needed", ws_bytes, p.ws_bytes));
        if ((uintptr_t)ws % 256) fail(RV_E_WORKSPACE, "workspace must be 256-byte aligned");
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) fail(RV_E_DEVICE, "no current HIP device");
    std::vector<void*>* fns = nullptr;
    ensure_loaded(p, dev, &fns);
    // every kernel parameter is a pointer: the kernel-argument block is the
    // packed array of them, handed over whole (no per-argument lookups)
    constexpr size_t kMaxParams = 64;
    for (size_t i = 0; i < p.kernels.size(); ++i) {
        const Kernel& k = p.kernels[i];
        if (k.plan == "empty" || k.grid[0] == 0) continue;
        const std::vector<Loc>& locs = p.kparams[i];
        if (locs.size() > kMaxParams) fail(RV_E_LAUNCH, fmt("kernel %s has %zu parameters", k.name.c_str(), locs.size()));
        void* ptrs[kMaxParams];
        for (size_t a = 0; a < locs.size(); ++a) {
            const Loc& L = locs[a];
            ptrs[a] = L.kind == 0 ? bufs[L.index].ptr
                      : L.kind == 1 ? bufs[nin + L.index].ptr
                                    : (void*)((char*)ws + p.regions[L.index].offset);
        }
        size_t arg_bytes = locs.size() * sizeof(void*);
        void* extra[] = {HIP_LAUNCH_PARAM_BUFFER_POINTER, ptrs, HIP_LAUNCH_PARAM_BUFFER_SIZE, &arg_bytes,
                         HIP_LAUNCH_PARAM_END};
        hipError_t e = hipModuleLaunchKernel((hipFunction_t)(*fns)[i], k.grid[0], k.grid[1], k.grid[2], k.block[0],
                                             k.block[1], k.block[2], 0, (hipStream_t)stream, nullptr, extra);
        if (e != hipSuccess)
            fail(RV_E_LAUNCH, fmt("launch of %s failed: %s", k.name.c_str(), hipGetErrorString(e)));
    }
}

}  // namespace rv
