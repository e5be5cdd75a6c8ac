"""Builds the reduce_view shared library in-tree.

The host code (graph intake, View algebra, scheduler, lowering, code
generation, runtime) is C++17 compiled by hipcc and linked against the HIP
runtime and the HIP runtime compiler; the device skeleton header is embedded
as a string and compiled per program for gfx950 at rv_compile time. A second
step compiles the device header for gfx950 with hipcc as a build check.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "_lib", "librv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HOST_SOURCES = ["view.cpp", "graph.cpp", "schedule.cpp", "lower.cpp", "codegen.cpp", "runtime.cpp", "codeobj.cpp",
                "abi.cpp"]
# hipcc flag set for any GPU code it compiles (packed FP32 instructions off)
GPU_FLAGS = ["--offload-arch=gfx950", "-O3", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _embed_header(out_dir: str) -> str:
    src = os.path.join(CSRC, "kernels", "rv_device.hpp")
    text = open(src).read()
    if ")RVHDR" in text:
        raise RuntimeError("device header contains the raw-string delimiter")
    path = os.path.join(out_dir, "rv_device_embed.cpp")
    body = ('// generated from csrc/kernels/rv_device.hpp\n'
            'namespace rv {\nextern const char* const kDeviceHeader;\n'
            'const char* const kDeviceHeader = R"RVHDR(' + text + ')RVHDR";\n}\n')
    if not os.path.exists(path) or open(path).read() != body:
        with open(path, "w") as f:
            f.write(body)
    return path


def check_device_header(verbose: bool = False) -> None:
    """Compiles the device skeleton (with a template instantiation of the
    contraction) for gfx950, so a broken skeleton fails the build here."""
    out_dir = os.path.join(HERE, "_build")
    os.makedirs(out_dir, exist_ok=True)
    tu = os.path.join(out_dir, "device_check.hip")
    with open(tu, "w") as f:
        f.write('#include <hip/hip_runtime.h>\n#include "%s"\n' % os.path.join(CSRC, "kernels", "rv_device.hpp"))
        f.write("struct E { __device__ float operator()(float a, int, int) const { return a; }\n"
                "  __device__ void store(int, int, float) const {} };\n"
                "#define K extern \"C\" __global__ void __launch_bounds__(256)\n"
                "K chk5(float* p) { p[0] = rv_fold_sum(p, 16); }\n"
                "extern \"C\" __global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) "
                "chk15(const unsigned short* a, const unsigned short* b, float* p) {\n"
                "  rv_gemm_w6_bf16<true, 1, E>(a, b, 0, 4096, 0, 4096, 4096, 4096, 4096, E{}, p); }\n"
                "extern \"C\" __global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) "
                "chk16(const unsigned short* a, const unsigned short* b, float* p) {\n"
                "  rv_gemm_w6_bf16<false, 0, E, 2>(a, b, 0, 4096, 0, 4096, 4096, 4096, 4096, E{}, p); }\n"
                "extern \"C\" __global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) "
                "chk17(const unsigned short* a, const unsigned short* b, float* p) {\n"
                "  rv_gemm_w6_bf16<true, 1, E, 1, true>(a, b, 0, 4104, 0, 4104, 4100, 4104, 4160, E{}, p, 4100, 4097); }\n"
                "extern \"C\" __global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) "
                "chk18(const unsigned short* a, const unsigned short* b, float* w) {\n"
                "  rv_gemm_w6_bf16<false, 0, rv_slice_epi, 1, false, 3, 1, 8>(a, b, 0, 8192, 0, 8192, 1024, 1024, 1024, "
                "rv_slice_epi{w, 1024}, nullptr, 1024, 1024); }\n"
                "K chk19(const float* w, float* p) { rv_gemm_slices<1, E>(w, 8, 1048576, 1000, 1000, E{}, p); }\n"
                "extern \"C\" __global__ void __launch_bounds__(256) chk12(const unsigned short* q, const unsigned short* k, const unsigned short* v, float* o, "
                "float* l) { rv_attn_fwd_bf16<32, true, false, 4>(q, k, v, o, l, 1000, 1000, 0.25f); }\n"
                "extern \"C\" __global__ void __launch_bounds__(256) chk13(const unsigned short* q, const unsigned short* k, const unsigned short* v, "
                "unsigned short* o, float* l) { rv_attn_fwd_bf16<64, false, true, 3>(q, k, v, o, l, 100, 333, 0.18f); }\n"
                "extern \"C\" __global__ void __launch_bounds__(256) chk14(const unsigned short* q, const unsigned short* k, const unsigned short* v, float* o, "
                "float* l) { rv_attn_fwd_bf16<128, true, false, 2>(q, k, v, o, nullptr, 130, 130, 0.1f); }\n")
    cmd = [HIPCC] + GPU_FLAGS + ["--cuda-device-only", "-c", tu, "-o", os.path.join(out_dir, "device_check.o")]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)


def build(verbose: bool = False) -> str:
    out_dir = os.path.join(HERE, "_build")
    os.makedirs(out_dir, exist_ok=True)
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    embed = _embed_header(out_dir)
    srcs = [os.path.join(CSRC, "host", s) for s in HOST_SOURCES] + [embed]
    # the library's own device workspace (a gfx950 device array): compiled as
    # HIP for gfx950, linked beside the host code
    scratch_o = os.path.join(out_dir, "scratch.o")
    cmd = [HIPCC] + GPU_FLAGS + ["-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include"), "-I",
                                 os.path.join(CSRC, "host"), "-c", os.path.join(CSRC, "host", "scratch.hip"),
                                 "-o", scratch_o]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    srcs += ["-x", "none", scratch_o]  # an object, whatever language the sources before it were taken as
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-O2", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wno-unused-function",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(CSRC, "host")] + srcs + [
           "-o", tmp, "-lhiprtc", "-Wl,-rpath,/opt/rocm/lib", "-Wl,--no-undefined"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    check_device_header(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
