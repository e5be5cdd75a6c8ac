// Internal graph, kernel plan and program structures of the library.
#pragma once

#include <cstdint>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "common.hpp"

namespace rv {

// ---------------------------------------------------------------------------
// graph intake (graph.cpp)
// ---------------------------------------------------------------------------
struct Node {
    int op = 0;
    int dtype = 0;
    int src[3] = {-1, -1, -1};
    int nsrc = 0;
    Shape shape;
    int slot = -1;        // BUFFER
    double cval = 0.0;    // CONST
    rv_view view{};       // VIEW (over src[0]'s row-major storage)
    uint32_t axes = 0;    // SUM / MAX
    // CUSTOM: kernel id, which of its outputs this node is, flags
    int custom = 0;
    int cout = 0;
    bool causal = false;
    // GATHER / SCATTER: the indexed axis; SCATTER: unordered atomic adds
    int axis = 0;
    bool atomic = false;
};

struct Graph {
    std::vector<Node> nodes;
    std::vector<int> outputs;
    int n_inputs = 0;
    std::vector<std::vector<int>> users;
};

Graph intake(const rv_node* nodes, int32_t n, const int32_t* outputs, int32_t nout);
bool is_elementwise(int op);
bool is_reduce(int op);
// A VIEW of a value of `src_shape` that only adds/removes size-1 dims and
// expands: each view dim either has stride 0 or walks one source dim of the
// same size, in order, with no offset and no mask. On success fills
// src_dim_of_view[d'] (source dim walked by view dim d', or -1).
bool pure_broadcast(const rv_view& v, const Shape& src_shape, std::vector<int>* src_dim_of_view);

// ---------------------------------------------------------------------------
// kernels (schedule.cpp / lower.cpp / codegen.cpp)
// ---------------------------------------------------------------------------
enum class KClass { EW, ROW, REDUCE, MFMA, FOLD, ATTN, SCATTER, SPLIT };
constexpr int EX_MFMA_ACC = 1000;  // Ex op: the contraction's accumulator at (m, n)
constexpr int EX_FOLD_ACC = 1001;  // Ex op: a split reduce's folded partials at this cell
const char* kclass_name(KClass k);

// Where a value lives in memory.
struct Loc {
    int kind = 0;  // 0 input slot, 1 output index, 2 workspace region
    int index = 0;
    bool operator==(const Loc& o) const { return kind == o.kind && index == o.index; }
};

// A load of one buffer through a View written over the kernel's iteration
// domain (ndim == domain rank, strides per domain dim).
struct Leaf {
    Loc loc;
    int dtype = RV_F32;
    rv_view v{};
    bool zero = false;  // every cell is outside the mask
};

// One value computed inside a kernel.
struct Ex {
    int op = 0;        // an rv_op; RV_BUFFER means "load leaf"
    int dtype = 0;     // dtype of the value (storage semantics)
    int a = -1, b = -1, c = -1;
    int leaf = -1;
    double cval = 0.0;
    uint32_t axes = 0;  // reduce dims (domain dims) for SUM/MAX
    bool stat = false;  // ROW kernels: constant along the reduced dims
    int node = -1;      // graph node this value came from (for describe)
    // GATHER: a = the index, leaf = the data at index g_lo along the
    // gathered axis (stride 0 there); the cell read is
    // leaf + (index - g_lo) * g_stride when g_lo <= index < g_hi, else zero
    int64_t g_stride = 0, g_lo = 0, g_hi = 0;
};

// One value the kernel writes: `ex` stored through view `v` (over the
// domain; reduced dims have stride 0) into `loc`.
struct Store {
    int ex = -1;
    Loc loc;
    int dtype = RV_F32;
    rv_view v{};
    int node = -1;
    int out_index = 0;  // ATTN: 0 the attention output, 1 the row logsumexp
};

struct Kernel {
    KClass cls = KClass::EW;
    std::string name;
    Shape domain;
    uint32_t rdims = 0;  // reduced domain dims (ROW / REDUCE / MFMA)
    std::vector<Leaf> leaves;
    std::vector<Ex> ex;
    std::vector<Store> stores;
    // lowering results
    std::string plan;        // "rowmajor", "tiled2d", "row", "cells", "gemm", "fold"
    std::string plan_json;   // extra plan fields for rv_describe
    int lane_dim = -1;       // innermost (thread-consecutive) domain dim
    unsigned grid[3] = {1, 1, 1};
    unsigned block[3] = {256, 1, 1};
    size_t lds = 0;
    // MFMA pattern (a, b: leaves of the bf16 operands; y: the contraction)
    int mfma_a = -1, mfma_b = -1, mfma_y = -1;
    bool mfma_partial = false;  // epilogue reduced to one partial per workgroup
    // extents the operand buffers hold (M, N >= 256, K a multiple of the kernel's k-step;
    // an operand that cannot be read in place is first copied, zero-padded,
    // into workspace); the domain keeps the output's (M, N, K)
    int64_t mfma_ext[3] = {0, 0, 0};
    bool mfma_copied[2] = {false, false};
    // split over k (mfma_split > 1 slices, kMfmaKStep-aligned): the slice
    // kernel stores every slice's raw float32 accumulators, [slice][m][n] over
    // the output's extents, in region slices_region; the kernel after it
    // (mfma_slices, plan "gemm_slices") sums them in slice order and runs the
    // epilogue
    int mfma_split = 1;
    bool mfma_slices = false;
    int slices_region = -1;
    // the kernel's schedule (chosen at lowering, baked in at codegen): the
    // MFMA / LDS-read / copy interleaving, and the copies issued in an even
    // / odd k-tile's first k16 step
    struct GemmSched {
        int pin = 1;
        int pe = 3, po = 1;
    } gemm;
    int partials_region = -1;   // workspace region of the partials
    int64_t n_partials = 0;
    // FOLD ("fold": the contraction's partials to one scalar; "fold_cells":
    // a split reduce's partials, fold_count per output cell, then the
    // region's elementwise tail on the folded value)
    int fold_src_region = -1;
    int64_t fold_count = 0;
    // SPLIT: the reduce (op, dtype) whose partials it writes; the matching
    // FOLD carries the same. split_pieces partials per output cell, laid out
    // cell-major ([cell][piece], split_row) or piece-major ([piece][cell],
    // split_cols) in region partials_region.
    int red_op = 0, red_dtype = 0;
    int64_t split_pieces = 0, split_cells = 0;
    bool split_cell_major = false;
    int64_t split_depth = 0;  // additions any term passes through in the partial
    int fold_cells_per_wg = 64;  // fold_cells over piece-major partials: cells per workgroup
    // ATTN (leaves q, k, v; domain (H, Tq, D); Tk = leaves[1].v.shape[1])
    double attn_scale = 0.0;
    bool attn_causal = false;
    // keys split into chunks of attn_chunk over workgroups (0: one
    // workgroup per query block); attn_map[w] = (query block << 16) | chunk;
    // chunk partials in workspace regions attn_reg_o, attn_reg_ml; the
    // merge kernel (attn_merge) folds them
    int64_t attn_chunk = 0;
    int attn_cmax = 1;
    std::vector<unsigned> attn_map;
    int attn_reg_o = -1, attn_reg_ml = -1;
    bool attn_merge = false;
    int attn_stages = 0;  // LDS stages of 64-key K/V tiles
    // SCATTER: one step of a scatter-add into `sc_out`. Domain: the index's
    // shape; ex sc_index / sc_values over it, sc_base over the output's.
    //   "atomic": every position adds its value with an atomic add (the
    //             target already holds the base)
    //   "keys":   one key per index cell: the target along the axis and
    //             the dims the index varies along (an index outside the axis
    //             gets the last key and a flagged cell id, and adds nothing)
    //   "hist", "scan": per-tile digit counts of a radix pass and their
    //             exclusive scan (only with more than kScanInline tiles;
    //             otherwise the move counts every tile itself)
    //   "move":   one stable 8-bit radix pass
    //   "bounds": the first sorted position of every key (its run is
    //             bounds[key] .. bounds[key + 1])
    //   "fold":   per target key, the base plus its run of sorted values
    //             folded in index order; every output cell written once
    std::string sc_part;
    int sc_index = -1, sc_values = -1, sc_base = -1;
    int sc_axis = 0;
    Loc sc_out;
    Shape sc_out_shape;
    int sc_dtype = RV_F32;
    uint32_t sc_fdims = 0;      // dims the index is constant along (carried)
    int64_t sc_cells = 0;       // index cells (positions with the carried dims at 0)
    int64_t sc_keys_n = 0;      // valid keys: out extent along the axis x varying dims
    int sc_pass = 0, sc_passes = 0;
    bool sc_fused_keys = false;  // first move computes the keys from the index (no keys kernel)
    int sc_reg_keys[2] = {-1, -1}, sc_reg_vals[2] = {-1, -1};
    int sc_reg_counts = -1;  // per-tile digit counts (more than kScanInline tiles)
    int sc_reg_bounds = -1;  // first sorted position of every key, and of key sc_keys_n
};

// Radix passes over at most this many tiles count their digits inside the
// move kernel (every workgroup counts every tile, in LDS).
constexpr int64_t kScanInline = 64;

struct Region {
    size_t offset = 0;
    size_t bytes = 0;
};

struct OutputInfo {
    Shape shape;
    int dtype = RV_F32;
    int node = -1;
};

struct Program {
    Graph g;
    std::vector<Kernel> kernels;
    std::vector<Region> regions;
    size_t ws_bytes = 0;
    std::vector<OutputInfo> outputs;
    std::vector<int64_t> input_nelems;  // required elements per input slot
    std::vector<int> input_dtype;
    std::string source;
    std::string options;
    std::string key;
    std::vector<char> code;  // gfx950 code object
    // per-device loaded module
    std::mutex mu;
    std::map<int, void*> modules;                        // device -> hipModule_t
    std::map<int, std::vector<void*>> functions;         // device -> hipFunction_t per kernel
    std::vector<std::vector<Loc>> kparams;               // kernel parameter order
};

// Register and memory budget of one compiled kernel (-1: not recorded).
struct KernelResources {
    int64_t vgpr = -1, agpr = -1, sgpr = -1, vgpr_spill = -1, sgpr_spill = -1;
    int64_t scratch = -1;  // private (scratch) bytes per lane
    int64_t lds = -1;      // static LDS bytes per workgroup
};
// Per kernel name, from the metadata note of a gfx950 code object.
std::map<std::string, KernelResources> kernel_resources(const std::vector<char>& code);

void schedule(Program& p);                 // fills kernels + regions
void lower(Program& p);                    // merges dims, picks plans and launch shapes
std::string codegen(const Program& p);     // HIP source of every kernel
std::string describe(const Program& p);    // JSON
void compile_code(Program& p);             // hiprtc -> p.code (runtime.cpp)
void launch(Program& p, const rv_buffer* bufs, int32_t nbufs, void* ws, size_t ws_bytes, void* stream);
// whether the program's code object is loaded on device `dev` (loading it
// allocates device memory; the first rv_launch on a device does it)
bool loaded_on(Program& p, int dev);
// The library's own workspace (scratch.hip): a device array of
// kScratchBytes per GPU, for callers that cannot allocate.
constexpr size_t kScratchBytes = (size_t)64 << 20;
void* scratch_ptr(int dev);
void launch_noalloc(Program& p, const rv_buffer* bufs, int32_t nbufs, void* stream);
void device_check(int device);

std::string json_view(const rv_view& v);
std::vector<Loc> kernel_param_locs(const Program& p, const Kernel& k);
// ROW kernels: (MAX, SUM) value pairs whose SUM adds EXP(X - MAX(X)) over
// float32, which the streaming plan folds in one pass with the online
// max/denominator recurrence.
std::vector<std::pair<int, int>> online_softmax_pairs(const Kernel& k);
// k-depth the contraction kernel steps by (its operands hold a multiple of
// it): 64, A being staged 64 deep.
constexpr int64_t kMfmaKStep = 64;
// Value `e` of kernel `k` is the same at every index along domain dim `d`.
bool ex_invariant(const Kernel& k, int e, int d);

}  // namespace rv
