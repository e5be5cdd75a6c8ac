// A library-owned workspace for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): one file-scope device array per GPU, sized kScratchBytes, held
// by every GPU the library runs on until the process ends. rv_launch_noalloc
// runs a program with it in place of a caller's workspace. Every call on a
// GPU shares that GPU's array and it keeps the last call's contents; no
// kernel of this library needs its workspace cleared first. Calls that
// overlap on one GPU (different streams, or different host threads) race on
// it.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "graph.hpp"

namespace rv {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The device address of this GPU's array. In host code `scratch` names a
// host-side stand-in, never the device memory: its address comes from the
// runtime, once per device, with that device current.
void* scratch_ptr(int dev) {
    static std::mutex mu;
    static std::map<int, void*> ptrs;
    std::lock_guard<std::mutex> lk(mu);
    auto it = ptrs.find(dev);
    if (it != ptrs.end()) return it->second;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur != dev) fail(RV_E_DEVICE, "scratch: the device is not current");
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
        fail(RV_E_DEVICE, fmt("hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e)));
    if ((uintptr_t)ptr % 256) fail(RV_E_DEVICE, "scratch is not 256-byte aligned");
    ptrs[dev] = ptr;
    return ptr;
}

void launch_noalloc(Program& p, const rv_buffer* bufs, int32_t nbufs, void* stream) {
    if (p.ws_bytes > kScratchBytes)
        fail(RV_E_WORKSPACE, fmt("the program needs %zu bytes of workspace; the library's own holds %zu", p.ws_bytes,
                                 kScratchBytes));
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) fail(RV_E_DEVICE, "no current HIP device");
    // loading the code object allocates device memory: this call only runs
    // programs already loaded on the device
    if (!loaded_on(p, dev))
        fail(RV_E_INVALID, fmt("rv_launch_noalloc: the program is not loaded on device %d yet (loading allocates "
                               "device memory; one rv_launch on that device loads it)",
                               dev));
    void* ws = p.ws_bytes ? scratch_ptr(dev) : nullptr;
    launch(p, bufs, nbufs, ws, p.ws_bytes ? kScratchBytes : 0, stream);
}

}  // namespace rv
