/*
 * rv.h -- C ABI of the reduce_view library: a lazy tensor-graph region
 * (elementwise primitives read through View index arithmetic, ending in SUM
 * or MAX) compiled into fused HIP kernels for MI355X (gfx950) and launched on
 * the caller's stream.
 *
 * Sources of the contract (cited by page title and section):
 *   - limn README, "Architecture": the graph is a DAG over a closed set of
 *     primitives, built lazily and run on demand; a View is
 *     (shape, strides, offset, mask) and reshape, permute, expand, pad and
 *     shrink compose into one View that lowers to index arithmetic.
 *   - limn README, "The op set": the primitive names and the seven dtypes.
 *   - limn README, "Reading the schedule": a cut falls wherever a value has to
 *     exist in memory; a reduce keeps its reduced dims with size 1.
 *   - limn README, "Backends": programs are cached; selecting a device whose
 *     toolchain is missing fails at selection with the reason.
 *   - limn README, "Adding one": a backend is one rendering of the IR plus
 *     hooks that move bytes.
 *   - Tiki README, "What works today": launches go through caller-owned
 *     buffers and stream.
 *   - Tiki README, "Compile model code": an unsupported operation, layout or
 *     device raises a typed error naming the contract; an explicit backend
 *     never silently runs another implementation.
 *   - Tiki README, "The architecture we want": schedules and register/LDS
 *     budgets are inspectable before launch (rv_describe).
 *   - Tiki README, "Milestones", gate 4: the cache identity covers source,
 *     compiler version and options, target, shapes/strides, dtype, constants,
 *     layout, schedule and calling convention.
 *
 * Conventions for every call:
 *   - No call throws; each returns an rv_status. On failure rv_last_error()
 *     returns a thread-local message naming the broken contract.
 *   - Views are in ELEMENTS, not bytes. mask_lo/mask_hi give a half-open
 *     range per dim; a cell outside the range reads zero and its address is
 *     never formed into a load. Strides must be >= 0 (a step other than 1
 *     has no View: limn README, "Architecture").
 *   - The caller owns all device memory (inputs, outputs, workspace) and the
 *     stream. The library never allocates device memory and never
 *     synchronises. It owns only rv_program objects and the code cache.
 */
#ifndef REDUCE_VIEW_RV_H
#define REDUCE_VIEW_RV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RV_MAX_DIMS 8

typedef enum rv_status {
    RV_OK = 0,
    RV_E_INVALID = -1,            /* malformed argument or graph */
    RV_E_UNSUPPORTED_OP = -2,     /* ASSIGN, an unknown CUSTOM kernel, a narrow atomic scatter */
    RV_E_UNSUPPORTED_LAYOUT = -3, /* e.g. a reshape that does not compose into one View */
    RV_E_DTYPE = -4,              /* dtype rule broken (mixed operands, EXP of an int, ...) */
    RV_E_OUT_OF_BOUNDS = -5,      /* a View can address outside its buffer */
    RV_E_WORKSPACE = -6,          /* workspace missing or too small */
    RV_E_DEVICE = -7,             /* no device, or not gfx950 */
    RV_E_COMPILE = -8,            /* the HIP runtime compiler rejected generated code */
    RV_E_LAUNCH = -9              /* a HIP call failed at launch */
} rv_status;

/* limn README, "The op set" (dtype paragraph): float16 and bfloat16 are
 * storage widths computed in float32; ints wrap modulo 2^width. */
typedef enum rv_dtype {
    RV_F32 = 0, RV_BF16 = 1, RV_F16 = 2, RV_F64 = 3, RV_I32 = 4, RV_I16 = 5, RV_I8 = 6
} rv_dtype;

/* limn README, "The op set". CMPLT yields RV_I8 0/1; WHERE treats a nonzero
 * condition as true. ASSIGN is declined with RV_E_UNSUPPORTED_OP; so is
 * CUSTOM unless it names RV_CUSTOM_SDPA_FWD. */
typedef enum rv_op {
    RV_BUFFER = 0, RV_CONST = 1, RV_VIEW = 2,
    RV_NEG = 3, RV_EXP = 4, RV_LOG = 5, RV_SQRT = 6, RV_RECIP = 7, RV_CAST = 8,
    RV_ADD = 9, RV_MUL = 10, RV_CMPLT = 11, RV_WHERE = 12,
    RV_SUM = 13, RV_MAX = 14, RV_CONTIGUOUS = 15,
    RV_GATHER = 16, RV_SCATTER = 17, RV_ASSIGN = 18, RV_CUSTOM = 19
} rv_op;

/* CUSTOM kernels (limn README, "The op set", escape hatch: a kernel the
 * device supplies whole; a kernel with several outputs is one node per
 * output, the nodes sharing their sources).
 *
 * RV_CUSTOM_SDPA_FWD, in `rv_node.buf`: fused attention forward (limn README,
 * "The op set": the forward saves one number per row besides the answer,
 * the logsumexp L; Tiki README, "Write the attention kernel at the
 * algorithm level": running maximum, denominator and accumulator per query
 * row over tiles of keys).
 *   src[0..2] = q (H, Tq, D), k (H, Tk, D), v (H, Tk, D), all RV_BF16, with
 *               D one of 32, 64, 128; H <= 65535.
 *   cval       = the score scale (finite and > 0; RV_E_INVALID otherwise).
 *   reduce_axes = RV_SDPA_CAUSAL (key j hidden from query i when j > i) OR'd
 *               with (output index << 16): output 0 is
 *               O = softmax(scale * q k^T) v, shape (H, Tq, D), dtype RV_F32 or
 *               RV_BF16; output 1 is L = the row logsumexp (max + log of the
 *               sum), shape (H, Tq, 1), RV_F32.
 * Nodes with the same sources, scale and causal flag are one kernel launch.
 * The probabilities enter the second contraction rounded to bfloat16 (the
 * matrix cores' operand type); the result agrees with the primitive
 * composition (scores, max-shifted softmax, contraction over keys) within
 * the bound that rounding implies. */
#define RV_CUSTOM_SDPA_FWD 1
#define RV_SDPA_CAUSAL 1u

/* Indexed ops (limn README, "The op set", indexed). `reduce_axes` holds
 * exactly one bit: the axis a.
 *   GATHER : src[0] = data, src[1] = index (RV_I32) shaped like data except
 *            along a. out[p] = data[p with coordinate a replaced by
 *            index[p]]; shape and a of the index, dtype of the data; an
 *            index outside [0, data extent along a) reads zero.
 *   SCATTER: src[0] = base, src[1] = index (RV_I32) shaped like base except
 *            along a, src[2] = values (the index's shape, the base's dtype).
 *            out = base, then values[p] is added at p with coordinate a
 *            replaced by index[p]; an index outside the axis drops its value.
 *            `buf` picks how colliding adds combine:
 *              RV_SCATTER_ORDERED: in ascending row-major order of p, each
 *                add rounded to the dtype (limn README, "Backends": the C
 *                device folds a scatter's colliding adds serially); the
 *                same bits on every run, every dtype;
 *              RV_SCATTER_ATOMIC: hardware atomic adds in whatever order
 *                they land (limn README, "Backends": the cuda device's
 *                scatter); f32, f64 and i32 only (RV_E_UNSUPPORTED_OP
 *                otherwise); ints are exact, floats agree with the ordered
 *                result up to the order of colliding adds.
 * The index must have fewer than 2^31 cells and every dim must fit in int32;
 * an ordered SCATTER also needs fewer than 2^31 target keys (the base's
 * extent along a times the index's extents along the dims the index varies
 * in besides a). RV_E_INVALID otherwise. */
#define RV_SCATTER_ORDERED 0
#define RV_SCATTER_ATOMIC 1

/* A View (limn README, "Architecture"): cell i of `shape` reads element
 * offset + sum_d i_d * strides[d] of its source's row-major storage when
 * mask_lo[d] <= i_d < mask_hi[d] for every d, and reads zero otherwise. */
typedef struct rv_view {
    int32_t ndim;
    int32_t reserved;
    int64_t shape[RV_MAX_DIMS];
    int64_t strides[RV_MAX_DIMS];
    int64_t offset;
    int64_t mask_lo[RV_MAX_DIMS];
    int64_t mask_hi[RV_MAX_DIMS];
} rv_view;

/* One graph node. Nodes are topologically ordered: src[] names earlier
 * nodes (unused entries -1).
 *   BUFFER : `buf` is the input slot; view = contiguous view of its shape.
 *   CONST  : cval of `dtype`, broadcast to view.shape.
 *   VIEW   : `view` over the row-major storage of src[0] (a BUFFER, a VIEW,
 *            or a computed value). A View of a computed value that is only a
 *            broadcast (size-1 dims added, then expanded) fuses; any other
 *            View of a computed value makes that value exist in memory first.
 *   CAST   : converts src[0] to `dtype` (float->float rounds to nearest even;
 *            float->int truncates toward zero).
 *   SUM/MAX: reduces the dims set in the bitmask `reduce_axes`, keeping them
 *            with size 1 (limn README, "Reading the schedule").
 * For every other op `dtype`, `buf`, `cval` and `view` are ignored (dtype and
 * shape are inferred). */
typedef struct rv_node {
    int32_t op;
    int32_t dtype;
    int32_t src[3];
    int32_t buf;
    uint32_t reduce_axes;
    int32_t reserved;
    double cval;
    rv_view view;
} rv_node;

/* A caller-owned device buffer. `nelems` counts elements of `dtype`. */
typedef struct rv_buffer {
    void* ptr;
    int64_t nelems;
    int32_t dtype;
    int32_t reserved;
} rv_buffer;

typedef struct rv_program rv_program;

/* Checks that `device` exists and is gfx950 (limn README, "Backends": fail at
 * selection with the reason). RV_E_DEVICE otherwise. */
rv_status rv_init(int device);

/* Validates the graph, infers shapes and dtypes, cuts it into kernels,
 * lowers every View to index arithmetic and compiles the kernels for gfx950
 * with the HIP runtime compiler (cached by source hash and options). Host
 * only: needs no device. `outputs` names nout nodes whose values the
 * program writes. On success *out owns a program to free with
 * rv_program_free. */
rv_status rv_compile(const rv_node* nodes, int32_t n, const int32_t* outputs, int32_t nout,
                     rv_program** out);

/* Shape (as a contiguous view) and dtype that node `i` of nodes[0..n) would
 * have, inferred by the same intake rv_compile runs (only nodes[0..i] are
 * read). Lets a caller compose a View over a computed value without
 * re-implementing shape inference. */
rv_status rv_node_shape(const rv_node* nodes, int32_t n, int32_t i, rv_view* shape, int32_t* dtype);

/* Number of input slots (1 + the largest BUFFER `buf`) and outputs. */
rv_status rv_program_io(const rv_program* prog, int32_t* n_inputs, int32_t* n_outputs);

/* Shape (as a contiguous view) and dtype of output `i`. */
rv_status rv_output_desc(const rv_program* prog, int32_t i, rv_view* shape, int32_t* dtype);

/* Bytes of device workspace rv_launch needs (0 if none). */
rv_status rv_workspace_size(const rv_program* prog, size_t* bytes);

/* Enqueues the program's kernels on `stream` (a hipStream_t; NULL is the
 * null stream) and returns without waiting. `bufs` holds n_inputs input
 * slots followed by n_outputs outputs (row-major, not aliasing any input).
 * Each buffer must hold at least the elements its nodes address, with the
 * declared dtype; `workspace` must be device memory of at least
 * rv_workspace_size bytes, 256-byte aligned. The first launch on a device
 * loads the code object on that (current) device. */
rv_status rv_launch(const rv_program* prog, const rv_buffer* bufs, int32_t nbufs,
                    void* workspace, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): rv_launch
 * with the library's own workspace in place of a caller's. That workspace is
 * one device array of RV_SCRATCH_BYTES per GPU, reserved when the library's
 * code is first loaded on the GPU and held until the process ends; this call
 * allocates nothing. A program needing more workspace than that fails with
 * RV_E_WORKSPACE before anything is enqueued, and a program whose code is not
 * yet loaded on the current device (loading allocates; the first rv_launch on
 * a device does it) fails with RV_E_INVALID. Every call on a GPU shares
 * that GPU's array and it keeps the last call's contents (no kernel here
 * needs it cleared); calls that overlap on one GPU (other streams, other
 * host threads) race on it. Buffers and stream as for rv_launch. */
#define RV_SCRATCH_BYTES ((size_t)64 << 20)
rv_status rv_launch_noalloc(const rv_program* prog, const rv_buffer* bufs, int32_t nbufs, void* stream);

/* Writes a JSON description of the program (kernel classes, lowered index
 * expressions, tile plans, launch shapes, LDS bytes, and per compiled kernel
 * its VGPR / AGPR / SGPR counts, spills, scratch and LDS bytes read from the
 * gfx950 code object) into out[0..cap), NUL
 * terminated. If `needed` is not NULL it receives the full length + 1.
 * Truncates silently when cap is too small. */
rv_status rv_describe(const rv_program* prog, char* out, size_t cap, size_t* needed);

/* Writes the generated HIP source of the program, like rv_describe. */
rv_status rv_source(const rv_program* prog, char* out, size_t cap, size_t* needed);

void rv_program_free(rv_program* prog);

/* Thread-local message of the last failing call on this thread ("" if none). */
const char* rv_last_error(void);

/* ---- View algebra (limn README, "Architecture"): each call composes one
 * movement op into an existing View, at no cost and without touching data.
 * `in` and `out` may alias. ---- */

/* Contiguous row-major view of `shape`. */
rv_status rv_view_contiguous(const int64_t* shape, int32_t ndim, rv_view* out);
/* Same cells in a new shape; RV_E_UNSUPPORTED_LAYOUT when the result is not
 * one View (e.g. merging dims whose strides do not chain, or reshaping
 * across a masked dim). */
rv_status rv_view_reshape(const rv_view* in, const int64_t* shape, int32_t ndim, rv_view* out);
/* out dim d is in dim perm[d]. */
rv_status rv_view_permute(const rv_view* in, const int32_t* perm, rv_view* out);
/* Size-1 dims become shape[d] with stride 0; other dims must match. */
rv_status rv_view_expand(const rv_view* in, const int64_t* shape, rv_view* out);
/* before[d]/after[d] >= 0 zero cells added on each side of dim d. */
rv_status rv_view_pad(const rv_view* in, const int64_t* before, const int64_t* after, rv_view* out);
/* Keeps cells lo[d] <= i_d < hi[d]. */
rv_status rv_view_shrink(const rv_view* in, const int64_t* lo, const int64_t* hi, rv_view* out);

#ifdef __cplusplus
}
#endif

#endif /* REDUCE_VIEW_RV_H */
