// View -> index lowering: turns each kernel's Views into the index arithmetic
// its HIP code runs, and picks the tile plan and launch shape.
//
// limn README, "Reading the schedule": views become index arithmetic inside
// the kernel; the innermost loop is the dim that is stride-1 in the most
// buffers (here: the dim consecutive lanes walk); a padded read is a range
// check, and cutting the innermost loop at the mask edges leaves pieces that
// are wholly inside or outside the pad (here: interior tiles run without
// range checks, edge tiles with them). Dims that chain in every View
// (stride[d] == size[d+1] * stride[d+1], both unmasked) are merged first, so
// e.g. a (4096, 4096) row-major chain runs as one flat loop.
#include <algorithm>
#include <cctype>
#include <cstdlib>

#include "graph.hpp"

namespace rv {

std::string json_view(const rv_view& v) {
    std::string s = "{\"shape\":[";
    for (int d = 0; d < v.ndim; ++d) s += (d ? "," : "") + std::to_string(v.shape[d]);
    s += "],\"strides\":[";
    for (int d = 0; d < v.ndim; ++d) s += (d ? "," : "") + std::to_string(v.strides[d]);
    s += "],\"offset\":" + std::to_string(v.offset) + ",\"mask_lo\":[";
    for (int d = 0; d < v.ndim; ++d) s += (d ? "," : "") + std::to_string(v.mask_lo[d]);
    s += "],\"mask_hi\":[";
    for (int d = 0; d < v.ndim; ++d) s += (d ? "," : "") + std::to_string(v.mask_hi[d]);
    return s + "]}";
}


// Rewrites every View of `k` for a new domain made of groups of old dims:
// groups[j] lists consecutive old dims (outermost first) forming new dim j.
static void regroup(Kernel& k, const std::vector<std::vector<int>>& groups) {
    auto apply = [&](rv_view& v) {
        rv_view o{};
        o.ndim = (int)groups.size();
        o.offset = v.offset;
        for (size_t j = 0; j < groups.size(); ++j) {
            int64_t size = 1;
            for (int d : groups[j]) size *= v.shape[d];
            int last = groups[j].back();
            o.shape[j] = size;
            o.strides[j] = v.strides[last];
            if (groups[j].size() == 1) {
                o.mask_lo[j] = v.mask_lo[last];
                o.mask_hi[j] = v.mask_hi[last];
            } else {
                o.mask_lo[j] = 0;
                o.mask_hi[j] = size;
            }
        }
        v = o;
    };
    for (auto& L : k.leaves) apply(L.v);
    for (auto& s : k.stores) apply(s.v);
    Shape dom;
    uint32_t rd = 0;
    for (size_t j = 0; j < groups.size(); ++j) {
        int64_t size = 1;
        for (int d : groups[j]) size *= k.domain[d];
        dom.push_back(size);
        if ((k.rdims >> groups[j][0]) & 1u) rd |= 1u << j;
    }
    k.domain = dom;
    k.rdims = rd;
}

static bool full_mask(const rv_view& v, int d) { return v.mask_lo[d] == 0 && v.mask_hi[d] == v.shape[d]; }

// Drops size-1 dims and merges adjacent dims that chain in every View.
static void merge_dims(Kernel& k) {
    const int r = (int)k.domain.size();
    std::vector<int> keep;
    for (int d = 0; d < r; ++d)
        if (k.domain[d] != 1) keep.push_back(d);
    if (keep.empty()) {
        // every dim has size 1: one cell; keep dim 0 as a size-1 loop
        if (r == 0) {
            k.domain = Shape{1};
            for (auto& L : k.leaves) {
                L.v.ndim = 1; L.v.shape[0] = 1; L.v.strides[0] = 0; L.v.mask_lo[0] = 0; L.v.mask_hi[0] = 1;
            }
            for (auto& s : k.stores) {
                s.v.ndim = 1; s.v.shape[0] = 1; s.v.strides[0] = 0; s.v.mask_lo[0] = 0; s.v.mask_hi[0] = 1;
            }
            return;
        }
        keep.push_back(0);
    }
    std::vector<std::vector<int>> groups;
    for (int d : keep) {
        if (!groups.empty()) {
            int p = groups.back().back();
            bool ok = ((k.rdims >> p) & 1u) == ((k.rdims >> d) & 1u);
            auto chain = [&](const rv_view& v) {
                return v.strides[p] == k.domain[d] * v.strides[d] && full_mask(v, p) && full_mask(v, d);
            };
            for (auto& L : k.leaves) ok = ok && (L.zero || chain(L.v));
            for (auto& s : k.stores) ok = ok && chain(s.v);
            if (ok) {
                groups.back().push_back(d);
                continue;
            }
        }
        groups.push_back({d});
    }
    regroup(k, groups);
}

// Leaf or store addresses stay inside their buffer for every in-mask cell.
static void prove_in_bounds(const Program& p, const Kernel& k) {
    auto cap = [&](const Loc& L, int dtype) -> int64_t {
        if (L.kind == 0) return p.input_nelems[L.index];
        if (L.kind == 1) return numel(p.outputs[L.index].shape);
        return (int64_t)(p.regions[L.index].bytes / dtype_size(dtype));
    };
    auto check = [&](const rv_view& v, const Loc& L, int dtype, const char* what) {
        int64_t lo, hi;
        if (!view_addr_range(v, &lo, &hi)) return;
        if (lo < 0 || hi >= cap(L, dtype))
            fail(RV_E_OUT_OF_BOUNDS, fmt("%s of kernel %s addresses [%lld, %lld] outside its %lld elements", what,
                                         k.name.c_str(), (long long)lo, (long long)hi, (long long)cap(L, dtype)));
    };
    for (auto& L : k.leaves)
        if (!L.zero && k.plan != "fold") check(L.v, L.loc, L.dtype, "a load");
    // a gathered read adds index * g_stride for an index in [g_lo, g_hi)
    for (auto& e : k.ex) {
        if (e.op != RV_GATHER || e.g_hi <= e.g_lo || k.leaves[e.leaf].zero) continue;
        const Leaf& L = k.leaves[e.leaf];
        int64_t lo, hi;
        if (!view_addr_range(L.v, &lo, &hi)) continue;
        const int64_t a = 0, b = (e.g_hi - 1 - e.g_lo) * e.g_stride;
        lo += std::min(a, b);
        hi += std::max(a, b);
        if (lo < 0 || hi >= cap(L.loc, L.dtype))
            fail(RV_E_OUT_OF_BOUNDS, fmt("a gathered load of kernel %s addresses [%lld, %lld] outside its %lld elements",
                                         k.name.c_str(), (long long)lo, (long long)hi, (long long)cap(L.loc, L.dtype)));
    }
    if (k.cls == KClass::SCATTER && cap(k.sc_out, k.sc_dtype) < numel(k.sc_out_shape))
        fail(RV_E_OUT_OF_BOUNDS, fmt("the scatter target of kernel %s is smaller than its shape", k.name.c_str()));
    for (auto& s : k.stores)
        if (k.plan != "fold" && !(k.cls == KClass::MFMA && k.mfma_partial)) check(s.v, s.loc, s.dtype, "a store");
}

std::vector<std::pair<int, int>> online_softmax_pairs(const Kernel& k) {
    std::vector<std::pair<int, int>> out;
    auto f32 = [&](int e) { return e >= 0 && k.ex[e].dtype == RV_F32; };
    for (size_t s = 0; s < k.ex.size(); ++s) {
        const Ex& S = k.ex[s];
        if (S.op != RV_SUM || !f32((int)s) || S.a < 0) continue;
        const Ex& Ex_ = k.ex[S.a];
        if (Ex_.op != RV_EXP || !f32(S.a) || Ex_.a < 0) continue;
        const Ex& A = k.ex[Ex_.a];
        if (A.op != RV_ADD || !f32(Ex_.a)) continue;
        for (int side = 0; side < 2; ++side) {
            const int X = side ? A.b : A.a, N = side ? A.a : A.b;
            if (X < 0 || N < 0 || k.ex[N].op != RV_NEG) continue;
            const int M = k.ex[N].a;
            if (M < 0 || k.ex[M].op != RV_MAX || k.ex[M].a != X || !f32(M) || !f32(X)) continue;
            if (k.ex[M].axes != S.axes) continue;
            out.emplace_back(M, (int)s);
            break;
        }
    }
    return out;
}

// Accumulator width of a reduce: float64 totals for float64, 4 bytes else
// (float32 for float32 and the half widths, a wrapping uint32 / int32 for
// the ints).
static int acc_bytes(int dtype) { return dtype == RV_F64 ? 8 : 4; }

// SPLIT plans. The reduce range (the reduced dims, row-major) is cut into P
// pieces; workgroup (cells, piece) folds its piece in a fixed order.
//   split_row  (a reduced dim is the one stride-1 in the most buffers): 256
//              lanes per (cell, piece), each lane VW consecutive elements of
//              U vectors per chunk of 256 * VW * U, chunks of a piece in
//              order; lane totals through a butterfly and the 4 waves in
//              order. Partials [cell][piece].
//   split_cols (a kept dim is): one lane per cell, 256 cells per
//              workgroup, the lane walks its piece's L reduce positions in
//              order. Partials [piece][cell].
// About 2048 workgroups (8 per CU), so each CU keeps enough loads in flight.
static void plan_split(Program& p, Kernel& k) {
    char buf[512];
    merge_dims(k);
    const int rank = (int)k.domain.size();
    int64_t C = 1, N = 1;
    for (int d = 0; d < rank; ++d) ((k.rdims >> d) & 1u ? N : C) *= k.domain[d];
    int best = -1, best_votes = -1;
    for (int d = 0; d < rank; ++d) {
        int votes = 0;
        for (auto& L : k.leaves)
            if (!L.zero && L.v.strides[d] == 1) ++votes;
        if (votes > best_votes || (votes == best_votes && d > best)) {
            best = d;
            best_votes = votes;
        }
    }
    const int64_t target = env_int("RV_SPLIT_WORKGROUPS", 2048);
    const bool rowp = (k.rdims >> best) & 1u;
    int64_t P, depth;
    if (rowp) {
        k.plan = "split_row";
        bool two = true, eight = false;
        for (auto& L : k.leaves)
            if (!L.zero) {
                bool along = false;
                for (int d = 0; d < rank; ++d)
                    if (((k.rdims >> d) & 1u) && L.v.strides[d] != 0) along = true;
                if (along && dtype_size(L.dtype) != 2) two = false;
                if (dtype_size(L.dtype) == 8) eight = true;
            }
        const int VW = two ? 8 : eight ? 2 : 4, U = 4, T = 256;
        const int64_t CH = (int64_t)T * VW * U, NCH = (N + CH - 1) / CH;
        P = std::max<int64_t>(1, std::min<int64_t>(NCH, (target + C - 1) / C));
        const int64_t CPP = (NCH + P - 1) / P;
        P = (NCH + CPP - 1) / CPP;
        k.grid[0] = (unsigned)(C * P);
        k.block[0] = T;
        k.lane_dim = best;
        k.lds = 4 * 8;
        // a lane's CPP * VW * U terms in order, 6 butterfly levels, 3 waves
        depth = CPP * VW * U - 1 + 6 + 3;
        snprintf(buf, sizeof buf, "\"threads_per_row\":%d,\"rows_per_block\":1,\"vec\":%d,\"unroll\":%d,"
                 "\"chunks\":%lld,\"row_len\":%lld,\"rows\":%lld,\"online\":[],\"pieces\":%lld,"
                 "\"chunks_per_piece\":%lld,\"partials\":\"cell-major\",\"sum_depth\":%lld",
                 T, VW, U, (long long)NCH, (long long)N, (long long)C, (long long)P, (long long)CPP,
                 (long long)depth);
        k.split_cell_major = true;
    } else {
        k.plan = "split_cols";
        const int64_t CT = (C + 255) / 256;
        P = std::max<int64_t>(1, std::min<int64_t>(N / 16, (target + CT - 1) / CT));
        const int64_t L = (N + P - 1) / P;
        P = (N + L - 1) / L;
        k.grid[0] = (unsigned)CT;
        k.grid[1] = (unsigned)P;
        k.block[0] = 256;
        k.lane_dim = best;
        depth = L - 1;
        snprintf(buf, sizeof buf, "\"cells\":%lld,\"lane_dim\":%d,\"reduce_len\":%lld,\"pieces\":%lld,"
                 "\"piece_len\":%lld,\"partials\":\"piece-major\",\"sum_depth\":%lld",
                 (long long)C, best, (long long)N, (long long)P, (long long)L, (long long)depth);
        k.split_cell_major = false;
    }
    k.split_pieces = P;
    k.split_cells = C;
    k.split_depth = depth;
    k.plan_json = buf;
    p.regions[k.partials_region].bytes = (size_t)(C * P * acc_bytes(k.red_dtype));
}

// FOLD of a split reduce: per output cell, the P partials in piece order
// (cell-major partials: a wave per cell, lanes take pieces l, l + 64, ... in
// order, then a butterfly; piece-major: a lane per cell), then the region's
// elementwise tail.
static void plan_fold_cells(Kernel& k, const Kernel& sp) {
    if (sp.split_cells >= ((int64_t)1 << 31)) fail(RV_E_INVALID, "internal: split reduce with 2^31 cells");
    char buf[512];
    k.plan = "fold_cells";
    k.fold_count = sp.split_pieces;
    k.split_pieces = sp.split_pieces;
    k.split_cells = sp.split_cells;
    k.split_cell_major = sp.split_cell_major;
    const int64_t C = sp.split_cells, P = sp.split_pieces;
    int64_t depth;
    if (k.split_cell_major) {  // a workgroup per cell: lane runs, butterfly, 4 waves
        k.grid[0] = (unsigned)C;
        depth = sp.split_depth + (P + 255) / 256 + 6 + 3;
    } else {
        // G cells per workgroup (a lane per cell, consecutive lanes on
        // consecutive cells), 256 / G lane groups each folding a run of the
        // pieces, the groups folded in order: G = 64, or fewer where that
        // leaves the CUs short of workgroups (4096 cells: G = 16, 256
        // workgroups)
        int G = 64;
        while (G > 16 && (C + G - 1) / G < 256) G /= 2;
        const int64_t groups = 256 / G, Q = (P + groups - 1) / groups;
        k.fold_cells_per_wg = G;
        k.grid[0] = (unsigned)((C + G - 1) / G);
        depth = sp.split_depth + Q + groups - 1;
    }
    k.lds = 4 * 64 * 8;
    k.block[0] = 256;
    k.lane_dim = (int)k.domain.size() - 1;
    snprintf(buf, sizeof buf,
             "\"partials\":%lld,\"cells\":%lld,\"src_region\":%d,\"layout\":\"%s\",\"cells_per_workgroup\":%d,"
             "\"sum_depth\":%lld",
             (long long)P, (long long)C, k.fold_src_region, k.split_cell_major ? "cell-major" : "piece-major",
             k.split_cell_major ? 1 : k.fold_cells_per_wg, (long long)depth);
    k.plan_json = buf;
}

static void plan_kernel(Program& p, Kernel& k, const Kernel* prev) {
    char buf[1024];
    switch (k.cls) {
        case KClass::SPLIT:
            plan_split(p, k);
            return;
        case KClass::FOLD: {
            if (prev && prev->cls == KClass::SPLIT) {
                plan_fold_cells(k, *prev);
                return;
            }
            k.plan = "fold";
            k.fold_count = prev ? prev->n_partials : 0;
            k.grid[0] = 1;
            k.block[0] = 256;
            k.lds = 256 * 4;
            snprintf(buf, sizeof buf, "\"partials\":%lld,\"src_region\":%d,\"sum_depth\":%lld",
                     (long long)k.fold_count, k.fold_src_region, (long long)((k.fold_count + 255) / 256 + 8));
            k.plan_json = buf;
            return;
        }
        case KClass::ATTN: {
            const int64_t H = k.domain[0], Tq = k.domain[1], D = k.domain[2];
            const int64_t Tk = k.leaves[1].v.shape[1];
            if (k.attn_merge) {  // D / 4 lanes per query, 256 / (D / 4) queries per workgroup
                k.plan = "attn_merge";
                k.grid[0] = (unsigned)((Tq + 127) / 128 * (128 / (256 / (D / 4))));
                k.grid[1] = (unsigned)H;
                k.block[0] = 256;
                k.lds = 0;
                snprintf(buf, sizeof buf, "\"key_chunk\":%lld,\"chunks_max\":%d,\"head_dim\":%lld",
                         (long long)k.attn_chunk, k.attn_cmax, (long long)D);
                k.plan_json = buf;
                return;
            }
            k.plan = "attn_fwd";
            // 128 queries (4 waves of 32) per workgroup, or one workgroup per
            // (query block, key chunk) when the keys are split
            k.grid[0] = k.attn_chunk > 0 ? (unsigned)k.attn_map.size() : (unsigned)((Tq + 127) / 128);
            k.grid[1] = (unsigned)H;
            // NS LDS stages of 64-key K and V tiles (RV_ATTN_STAGES, 2 to 4):
            // 3 at head width 32 (24 KB) and 64 (48 KB), 2 at 128 (64 KB),
            // so that several workgroups share a CU. Measured at 6 x 8192 x
            // 32, causal: 2, 3 and 4 stages within 2% of each other.
            const int NS = env_int("RV_ATTN_STAGES", D == 128 ? 2 : 3);
            if (NS < 2 || NS > 4) fail(RV_E_INVALID, "RV_ATTN_STAGES must be 2, 3 or 4");
            k.attn_stages = NS;
            k.block[0] = 256;
            k.lds = (size_t)NS * 2 * 64 * D * 2;
            snprintf(buf, sizeof buf,
                     "\"queries_per_workgroup\":128,\"queries_per_wave\":32,\"key_tile\":64,\"stages\":%d,"
                     "\"key_chunk\":%lld,\"chunks_max\":%d,"
                     "\"head_dim\":%lld,"
                     "\"keys\":%lld,\"causal\":%s,\"scale\":%.17g,\"mfma\":\"v_mfma_f32_32x32x16_bf16\","
                     "\"scores\":\"transposed (K q^T): one query per lane pair\",\"p_operand\":\"bf16\","
                     "\"tile_copy\":\"global_load_lds_dwordx4, XOR-swizzled chunks\",\"rescale_when_tile_sum_over\":256",
                     NS, (long long)k.attn_chunk, k.attn_cmax, (long long)D, (long long)Tk,
                     k.attn_causal ? "true" : "false", k.attn_scale);
            k.plan_json = buf;
            return;
        }
        case KClass::MFMA: {
            // 256 x 256 tiles, 4 waves of 128 x 128, operands copied straight
            // into LDS (kernels/rv_device.hpp), over the extents the operand
            // buffers hold (a ragged last tile is shifted back inside them),
            // tiles in XCD-contiguous order: A staged 64 deep in 3 stages, B
            // 32 deep in 4; pe / po copies issued in an even / odd k-tile's
            // first k16 step (RV_GEMM_W6_PE, RV_GEMM_W6_PO); the MFMA / LDS /
            // copy interleaving (RV_GEMM_PIN: 1 pinned, 2 reads front-loaded,
            // 0 free). Measured on cold 4096^3 operands: 105 us (the same
            // tiles staged 32 deep in 4 or 5 stages took 112 us at best).
            const int64_t M = k.domain[0], N = k.domain[1];
            const int64_t Me = k.mfma_ext[0], Ne = k.mfma_ext[1], Ke = k.mfma_ext[2];
            const int S = k.mfma_split;
            if (k.mfma_slices) {
                // the slices' fold: 4 consecutive cells a lane, each the S
                // planes in slice order, then the epilogue; a partial adds a
                // lane's 4 cells, 6 butterfly levels and 3 cross-wave
                // additions (the slices' own sum is part of the contraction)
                const int64_t cells = M * N;
                k.plan = "gemm_slices";
                k.grid[0] = (unsigned)((cells + 1023) / 1024);
                k.block[0] = 256;
                k.lds = 16;
                k.n_partials = k.grid[0];
                snprintf(buf, sizeof buf,
                         "\"split_k\":%d,\"slices_region\":%d,\"plane\":%lld,\"cells_per_lane\":4,"
                         "\"partial_sum_depth\":%d",
                         S, k.slices_region, (long long)((cells + 63) / 64 * 64), 3 + 6 + 3);
                k.plan_json = buf;
                if (k.mfma_partial) {
                    p.regions[k.partials_region].bytes = (size_t)k.n_partials * 4;
                    k.stores[0].loc = Loc{2, k.partials_region};
                }
                return;
            }
            const int pin = std::max(0, std::min(2, env_int("RV_GEMM_PIN", 1)));
            const int pe = std::max(0, std::min(12, env_int("RV_GEMM_W6_PE", 3)));
            const int po = std::max(0, std::min(4, env_int("RV_GEMM_W6_PO", 1)));
            k.plan = "gemm_w6";
            k.gemm.pin = pin;
            k.gemm.pe = pe;
            k.gemm.po = po;
            k.lds = 3 * 256 * 64 * 2 + 4 * 256 * 32 * 2;
            const int64_t tiles = ((Me + 255) / 256) * ((Ne + 255) / 256);
            if (tiles >= ((int64_t)1 << 31)) fail(RV_E_UNSUPPORTED_LAYOUT, "contraction of 2^31 or more output tiles");
            k.grid[0] = (unsigned)(tiles * S);
            k.block[0] = 256;
            k.n_partials = k.grid[0];
            const bool kn = k.leaves[k.mfma_b].v.strides[1] == 1;
            const bool ragged = Me % 256 || Ne % 256 || Me != M || Ne != N;
            char stage_buf[160];
            snprintf(stage_buf, sizeof stage_buf,
                     "\"stages\":{\"A\":3,\"B\":4},\"stage_depth\":{\"A\":64,\"B\":32},"
                     "\"early_copies\":[%d,%d]",
                     pe, po);
            // per lane: 256 values summed in order, 6 butterfly levels, 3
            // cross-wave additions; the fold adds its own depth
            snprintf(buf, sizeof buf,
                     "\"tile\":[256,256,32],\"waves\":4,\"wave_tiles\":[4,4],\"mfma\":\"v_mfma_f32_32x32x16_bf16\","
                     "\"b_layout\":\"%s\",\"xcd_remap\":8,\"partial_sum_depth\":%d,%s,"
                     "\"interleave\":%d,\"extent\":[%lld,%lld,%lld],\"ragged\":%s,"
                     "\"copied\":{\"A\":%s,\"B\":%s},\"operand_leaves\":[%d,%d],\"split_k\":%d,"
                     "\"slices_region\":%d",
                     kn ? "kn" : "nk", 256 - 1 + 6 + 3, stage_buf, pin, (long long)Me, (long long)Ne, (long long)Ke,
                     ragged ? "true" : "false", k.mfma_copied[0] ? "true" : "false", k.mfma_copied[1] ? "true" : "false",
                     k.mfma_a, k.mfma_b, S, k.slices_region);
            k.plan_json = buf;
            if (k.mfma_partial) {
                p.regions[k.partials_region].bytes = (size_t)k.n_partials * 4;
                k.stores[0].loc = Loc{2, k.partials_region};
            }
            return;
        }
        case KClass::SCATTER: {
            const int64_t cells = k.sc_cells, nb = (cells + 2047) / 2048;
            const int64_t nf = k.sc_cells ? numel(k.domain) / k.sc_cells : 0;
            k.plan = "scatter_" + k.sc_part;
            k.block[0] = 256;
            auto cap_grid = [](int64_t g) { return (unsigned)std::max<int64_t>(1, std::min<int64_t>(g, 1 << 20)); };
            // lanes per key: enough for the carried cells, CB consecutive
            // cells per lane when the last dim is carried and CB divides it
            const int last = (int)k.domain.size() - 1;
            const int vcb = std::max(1, std::min(4, 16 / dtype_size(k.sc_dtype)));
            const bool vec = ((k.sc_fdims >> last) & 1u) && vcb > 1 && k.domain[last] % vcb == 0;
            int tps = 1;
            while (tps < 256 && tps * (vec ? vcb : 1) < nf) tps *= 2;
            if (k.sc_part == "atomic") {
                k.grid[0] = cap_grid((numel(k.domain) + 255) / 256);
            } else if (k.sc_part == "keys") {
                k.grid[0] = cap_grid((cells + 255) / 256);
            } else if (k.sc_part == "hist") {
                k.grid[0] = (unsigned)nb;
                k.lds = 256 * 4;
            } else if (k.sc_part == "move") {  // 16 waves per tile
                k.grid[0] = (unsigned)nb;
                k.block[0] = 1024;
                k.lds = (256 + 16 * 256 + 16 + (nb <= kScanInline ? 256 * 64 : 0)) * 4;
            } else if (k.sc_part == "scan") {
                k.grid[0] = 256;
            } else if (k.sc_part == "bounds") {  // a wave per 64 sorted positions, one more past the end
                k.grid[0] = cap_grid((cells / 64 + 1 + 3) / 4);
            }
            // fold: a group of tps lanes takes R keys at a time
            const int R = env_int("RV_SCATTER_R", 4);
            if (R < 1 || R > 16) fail(RV_E_INVALID, "RV_SCATTER_R must be in 1..16");
            const int64_t kpb = (int64_t)R * (256 / tps);
            if (k.sc_part == "fold") k.grid[0] = cap_grid((k.sc_keys_n + kpb - 1) / kpb);
            snprintf(buf, sizeof buf,
                     "\"part\":\"%s\",\"axis\":%d,\"carried_dims\":%u,\"index_cells\":%lld,\"keys\":%lld,"
                     "\"radix_passes\":%d,\"pass\":%d,\"tile\":2048,\"tiles\":%lld,\"scan_inline\":%s,"
                     "\"lanes_per_key\":%d,\"keys_per_group\":%d,\"keys_per_workgroup\":%lld,\"ordered\":%s",
                     k.sc_part.c_str(), k.sc_axis, k.sc_fdims, (long long)cells, (long long)k.sc_keys_n, k.sc_passes,
                     k.sc_pass, (long long)nb, nb <= kScanInline ? "true" : "false", tps, R, (long long)kpb,
                     k.sc_part == "atomic" ? "false" : "true");
            k.plan_json = buf;
            if (k.sc_part == "move") k.plan_json += k.sc_fused_keys ? ",\"keys_from_index\":true" : "";
            return;
        }
        default: break;
    }
    merge_dims(k);
    const int rank = (int)k.domain.size();
    // nothing to compute unless a reduce over an empty range still has
    // cells to write (each gets the reduce identity, limn README, "The op
    // set": a reduce starts from its identity)
    bool any_store = false;
    for (auto& s : k.stores) {
        int64_t cells = 1;  // a reduced dim (stride 0 in the store) counts once
        for (int d = 0; d < s.v.ndim; ++d)
            if (!(((k.rdims >> d) & 1u) && s.v.strides[d] == 0)) cells *= s.v.shape[d];
        any_store = any_store || cells > 0;
    }
    if (numel(k.domain) == 0 && !any_store) {
        k.plan = "empty";
        k.grid[0] = 0;
        return;
    }
    if (k.cls == KClass::EW) {
        const int X = rank - 1, Y = rank - 2;
        bool tiled = false, gathers = false;
        for (auto& e : k.ex) gathers = gathers || e.op == RV_GATHER;
        if (rank >= 2 && k.domain[X] >= 8 && k.domain[Y] >= 8 && !gathers)
            for (auto& L : k.leaves)
                if (!L.zero && L.v.strides[Y] == 1 && L.v.strides[X] != 1) tiled = true;
        k.lane_dim = X;
        if (tiled) {
            k.plan = "tiled2d";
            // waves stacked WY (along Y) x WX (along X); 8 x 8 lanes of 4 x 4 cells each
            int WY = env_int("RV_EW_WAVES_Y", 1);
            if (WY != 1 && WY != 2 && WY != 4) fail(RV_E_INVALID, "RV_EW_WAVES_Y must be 1, 2 or 4");
            int WX = 4 / WY;
            // tile order: x-major, or diagonal when every streamed operand is
            // read transposed (a pure transpose: consecutive workgroups then
            // read different source columns instead of the same ones, 2.6%
            // faster on 4096^2; the chains with a row-major operand are not)
            bool all_t = true;
            for (auto& L : k.leaves)
                if (!L.zero && (L.v.strides[X] != 0 || L.v.strides[Y] != 0) &&
                    !(L.v.strides[Y] == 1 && L.v.strides[X] != 1))
                    all_t = false;
            int order = env_int("RV_EW_ORDER", all_t ? 2 : 0);
            int64_t B = numel(k.domain) / (k.domain[X] * k.domain[Y]);
            int64_t gx = (k.domain[X] + 32 * WX - 1) / (32 * WX), gy = (k.domain[Y] + 32 * WY - 1) / (32 * WY);
            k.grid[0] = (unsigned)(gx * gy);
            k.grid[1] = 1;
            k.grid[2] = (unsigned)B;
            k.block[0] = 256;
            // operands read along Y are transposed in registers: each lane
            // loads 4 vectors along Y and uses them as the columns of its
            // 4 x 4 block (an LDS-staged transpose measured 2% slower)
            int nt = 0;
            for (auto& L : k.leaves)
                if (!L.zero && L.v.strides[Y] == 1 && L.v.strides[X] != 1) ++nt;
            k.lds = 0;
            snprintf(buf, sizeof buf, "\"tile\":[%d,%d],\"waves\":[%d,%d],\"order\":%d,\"lane_block\":[4,4],"
                     "\"register_transposed_leaves\":%d", 32 * WY, 32 * WX, WY, WX, order, nt);
        } else {
            k.plan = "rowmajor";
            int maxsz = 1;
            for (auto& s : k.stores) maxsz = std::max(maxsz, dtype_size(s.dtype));
            // 16-byte accesses per lane; about 32 cells of every value in
            // flight per lane (2 vectors of int8, 4 of the wider types)
            int vw = std::max(1, std::min(16, 16 / maxsz));
            int64_t cpr = (k.domain[X] + vw - 1) / vw;
            int64_t chunks = cpr * (numel(k.domain) / k.domain[X]);
            // 4-byte cells that are read and written: one vector per lane
            // per grid step (measured 2-3% faster than 4 on the 4096^2 copy
            // and the embedding gather; a pure fill keeps 4, 7% faster)
            bool reads = false;
            for (auto& L : k.leaves)
                if (!L.zero) reads = true;
            int U = vw == 4 && reads ? 1 : std::max(1, std::min(4, 32 / vw));
            U = env_int("RV_EW_UNROLL", U);
            if (U < 1 || U > 16) fail(RV_E_INVALID, "RV_EW_UNROLL must be in 1..16");
            const int64_t cap = env_int("RV_EW_GRID_CAP", 256 * 32);
            if (cap < 1) fail(RV_E_INVALID, "RV_EW_GRID_CAP must be positive");
            int64_t blocks = (chunks + 256 * U - 1) / (256 * U);
            k.grid[0] = (unsigned)std::max<int64_t>(1, std::min<int64_t>(blocks, cap));
            k.block[0] = 256;
            snprintf(buf, sizeof buf, "\"vec\":%d,\"unroll\":%d,\"chunks\":%lld", vw, U, (long long)chunks);
        }
        k.plan_json = buf;
        return;
    }
    if (k.cls == KClass::ROW) {
        k.plan = "row";
        int64_t NR = 1, NK = 1;
        for (int d = 0; d < rank; ++d) ((k.rdims >> d) & 1u ? NR : NK) *= k.domain[d];
        bool two = true;
        for (auto& L : k.leaves)
            if (!L.zero && dtype_size(L.dtype) != 2) {
                bool along = false;
                for (int d = 0; d < rank; ++d)
                    if (((k.rdims >> d) & 1u) && L.v.strides[d] != 0) along = true;
                if (along) two = false;
            }
        for (auto& s : k.stores)
            if (dtype_size(s.dtype) != 2) {
                bool along = false;
                for (int d = 0; d < rank; ++d)
                    if (((k.rdims >> d) & 1u) && s.v.strides[d] != 0) along = true;
                if (along) two = false;
            }
        // 16-byte accesses: 8 cells of 2 bytes, 4 of 4, 2 of 8 (with 32-byte
        // float64 accesses each wave-wide store covered half lines and the
        // write traffic came out 5% above the bytes written)
        bool eight = false;
        for (auto& L : k.leaves)
            if (!L.zero && dtype_size(L.dtype) == 8) eight = true;
        for (auto& st : k.stores)
            if (dtype_size(st.dtype) == 8) eight = true;
        int vw = two ? 8 : eight ? 2 : 4;
        // about 64 bytes per lane of each row-long operand (16 cells of 4
        // bytes or more, 32 of 2 bytes): enough bytes in flight per lane, few
        // enough VGPRs for high occupancy (16 two-byte cells per lane left
        // RMSNorm over float16 rows 17% slower); never so few lanes that a
        // lane holds more than 32 cells, the most kept in registers
        const int cells = two ? 32 : 16;
        int T = 1024;
        while (T > 16 && (int64_t)T * cells > NR) T /= 2;
        while (T < 1024 && (NR + (int64_t)T * vw - 1) / ((int64_t)T * vw) * vw > 32) T *= 2;
        T = env_int("RV_ROW_THREADS", T);
        if (T < 1 || T > 1024 || (T & (T - 1))) fail(RV_E_INVALID, "RV_ROW_THREADS must be a power of two <= 1024");
        const int block = std::max(256, T);
        int rpw = block / T;
        int64_t nrg = (NK + rpw - 1) / rpw;
        // A row-long leaf that is the same for every row (a norm's weights)
        // is loaded once per workgroup; then the grid is persistent, two
        // workgroups per CU, each loading its next row group while it
        // reduces the current one. Otherwise one workgroup per row group
        // (measured faster without reused weights). RV_ROW_PREFETCH=0/1 and
        // RV_ROW_GRID override.
        bool reused = false;
        for (auto& L : k.leaves) {
            if (L.zero) continue;
            bool along = false, across = false;
            for (int d = 0; d < rank; ++d) {
                const bool red = (k.rdims >> d) & 1u;
                const bool m = !full_mask(L.v, d);
                if (red && (L.v.strides[d] != 0 || m)) along = true;
                if (!red && k.domain[d] > 1 && (L.v.strides[d] != 0 || m)) across = true;
            }
            if (along && !across) reused = true;
        }
        const bool prefetch = env_int("RV_ROW_PREFETCH", reused ? 1 : 0) != 0;
        k.grid[0] = (unsigned)std::max<int64_t>(
            1, std::min<int64_t>(nrg, env_int("RV_ROW_GRID", prefetch ? 2 * 256 : 1 << 30)));
        k.block[0] = (unsigned)block;
        k.lane_dim = rank - 1;
        int nv = (int)((NR + (int64_t)T * vw - 1) / ((int64_t)T * vw));
        // a row longer than about 32 cells per lane at 1024 lanes does not
        // fit in registers: stream it (RV_ROW_STREAM=1 forces, =0 forbids)
        const int stream_env = env_int("RV_ROW_STREAM", -1);
        if (stream_env == 1 || (stream_env != 0 && (int64_t)nv * vw > 32)) {
            k.plan = "row_stream";
            const int U = 4;
            k.grid[0] = (unsigned)std::max<int64_t>(1, std::min<int64_t>(nrg, env_int("RV_ROW_GRID", 1 << 30)));
            k.block[0] = (unsigned)block;
            k.lane_dim = rank - 1;
            const int64_t ch = (int64_t)T * vw * U;
            const auto pairs = online_softmax_pairs(k);
            int nred = 0;
            for (auto& e : k.ex)
                if (e.op == RV_SUM || e.op == RV_MAX) ++nred;
            k.lds = T > 64 ? (size_t)(nred + pairs.size()) * rpw * (T / 64) * 4 : 0;
            std::string on = "[";
            for (size_t i = 0; i < pairs.size(); ++i)
                on += fmt("%s[%d,%d]", i ? "," : "", pairs[i].first, pairs[i].second);
            on += "]";
            snprintf(buf, sizeof buf, "\"threads_per_row\":%d,\"rows_per_block\":%d,\"vec\":%d,\"unroll\":%d,"
                     "\"chunks\":%lld,\"row_len\":%lld,\"rows\":%lld,\"online\":%s", T, rpw, vw, U,
                     (long long)((NR + ch - 1) / ch), (long long)NR, (long long)NK, on.c_str());
            k.plan_json = buf;
            return;
        }
        int nred = 0;
        for (auto& e : k.ex)
            if (e.op == RV_SUM || e.op == RV_MAX) ++nred;
        k.lds = T > 64 ? (size_t)nred * rpw * (T / 64) * 4 : 0;
        snprintf(buf, sizeof buf, "\"threads_per_row\":%d,\"rows_per_block\":%d,\"vec\":%d,\"chunks\":%d,"
                 "\"row_len\":%lld,\"rows\":%lld,\"prefetch\":%d", T, rpw, vw, nv, (long long)NR, (long long)NK,
                 prefetch ? 1 : 0);
        k.plan_json = buf;
        return;
    }
    // REDUCE: one lane per output cell; lanes walk the kept dim that is
    // stride-1 in the most buffers (a tie keeps the later dim)
    k.plan = "cells";
    int best = -1, best_votes = -1;
    for (int d = 0; d < rank; ++d) {
        if ((k.rdims >> d) & 1u) continue;
        int votes = 0;
        for (auto& L : k.leaves)
            if (!L.zero && L.v.strides[d] == 1) ++votes;
        for (auto& s : k.stores)
            if (s.v.strides[d] == 1) ++votes;
        if (votes >= best_votes) {
            best = d;
            best_votes = votes;
        }
    }
    k.lane_dim = best;
    int64_t cells = 1;
    for (int d = 0; d < rank; ++d)
        if (!((k.rdims >> d) & 1u)) cells *= k.domain[d];
    k.grid[0] = (unsigned)std::max<int64_t>(1, std::min<int64_t>((cells + 255) / 256, 1 << 20));
    k.block[0] = 256;
    snprintf(buf, sizeof buf, "\"cells\":%lld,\"lane_dim\":%d", (long long)cells, best);
    k.plan_json = buf;
}

void lower(Program& p) {
    const Graph& g = p.g;
    p.input_nelems.assign(g.n_inputs, 0);
    p.input_dtype.assign(g.n_inputs, -1);
    for (const Node& nd : g.nodes) {
        if (nd.op != RV_BUFFER) continue;
        int64_t ne = numel(nd.shape);
        if (p.input_dtype[nd.slot] >= 0 && p.input_dtype[nd.slot] != nd.dtype)
            fail(RV_E_DTYPE, fmt("input slot %d is declared with two dtypes", nd.slot));
        p.input_dtype[nd.slot] = nd.dtype;
        p.input_nelems[nd.slot] = std::max(p.input_nelems[nd.slot], ne);
    }
    p.outputs.clear();
    for (int o : g.outputs) p.outputs.push_back(OutputInfo{g.nodes[o].shape, g.nodes[o].dtype, o});
    for (size_t i = 0; i < p.kernels.size(); ++i) plan_kernel(p, p.kernels[i], i ? &p.kernels[i - 1] : nullptr);
    size_t off = 0;
    for (auto& r : p.regions) {
        r.offset = off;
        off += (r.bytes + 255) / 256 * 256;
    }
    p.ws_bytes = off;
    // kernel names say what they are (class, plan, a hash of the lowered
    // kernel) so profiles of different programs can be told apart
    for (size_t i = 0; i < p.kernels.size(); ++i) {
        Kernel& k = p.kernels[i];
        std::string sig = std::string(kclass_name(k.cls)) + k.plan + k.plan_json;
        for (int64_t d : k.domain) sig += "," + std::to_string(d);
        for (auto& L : k.leaves) sig += json_view(L.v) + dtype_name(L.dtype);
        for (auto& st : k.stores) sig += json_view(st.v) + dtype_name(st.dtype);
        for (auto& e : k.ex)
            sig += fmt("|%d,%d,%d,%d,%d,%d,%.17g,%lld,%lld,%lld", e.op, e.dtype, e.a, e.b, e.c, e.leaf, e.cval,
                       (long long)e.g_stride, (long long)e.g_lo, (long long)e.g_hi);
        if (k.cls == KClass::SCATTER)
            sig += fmt("|%d,%d,%d,%d,%d,%d,%d,%d", k.sc_index, k.sc_values, k.sc_base, k.sc_out.kind, k.sc_out.index,
                       k.sc_dtype, k.sc_passes, k.sc_pass) + shape_str(k.sc_out_shape);
        uint64_t h = 1469598103934665603ull;
        for (unsigned char ch : sig) {
            h ^= ch;
            h *= 1099511628211ull;
        }
        std::string cls = kclass_name(k.cls);
        for (auto& ch : cls) ch = (char)tolower(ch);
        k.name = fmt("rv_%s_%s_%08x_%zu", cls.c_str(), k.plan.c_str(), (unsigned)(h & 0xffffffffu), i);
    }
    for (auto& k : p.kernels) prove_in_bounds(p, k);
}

// ---------------------------------------------------------------------------
// rv_describe
// ---------------------------------------------------------------------------
static std::string json_loc(const Loc& L) {
    static const char* kinds[] = {"input", "output", "workspace"};
    return fmt("{\"kind\":\"%s\",\"index\":%d}", kinds[L.kind], L.index);
}

std::string describe(const Program& p) {
    const std::map<std::string, KernelResources> res = kernel_resources(p.code);
    std::string s = "{\"n_inputs\":" + std::to_string(p.g.n_inputs) + ",\"workspace_bytes\":" +
                    std::to_string(p.ws_bytes) + ",\"cache_key\":\"" + p.key + "\",\"kernels\":[";
    for (size_t i = 0; i < p.kernels.size(); ++i) {
        const Kernel& k = p.kernels[i];
        if (i) s += ",";
        s += "{\"name\":\"" + k.name + "\",\"class\":\"" + kclass_name(k.cls) + "\",\"plan\":\"" + k.plan +
             "\",\"domain\":[";
        for (size_t d = 0; d < k.domain.size(); ++d) s += (d ? "," : "") + std::to_string(k.domain[d]);
        s += "],\"reduce_dims\":[";
        bool first = true;
        for (size_t d = 0; d < k.domain.size(); ++d)
            if ((k.rdims >> d) & 1u) {
                s += (first ? "" : ",") + std::to_string(d);
                first = false;
            }
        s += "],\"lane_dim\":" + std::to_string(k.lane_dim);
        s += fmt(",\"grid\":[%u,%u,%u],\"block\":[%u,%u,%u],\"lds_bytes\":%zu", k.grid[0], k.grid[1], k.grid[2],
                 k.block[0], k.block[1], k.block[2], k.lds);
        if (!k.plan_json.empty()) s += ",\"plan_detail\":{" + k.plan_json + "}";
        // the compiled kernel's budget (Tiki README, "The architecture we
        // want": visible before launch)
        auto r = res.find(k.name);
        if (r != res.end())
            s += fmt(",\"resources\":{\"vgpr\":%lld,\"agpr\":%lld,\"sgpr\":%lld,\"vgpr_spill\":%lld,"
                     "\"sgpr_spill\":%lld,\"scratch_bytes\":%lld,\"lds_bytes\":%lld}",
                     (long long)r->second.vgpr, (long long)r->second.agpr, (long long)r->second.sgpr,
                     (long long)r->second.vgpr_spill, (long long)r->second.sgpr_spill, (long long)r->second.scratch,
                     (long long)r->second.lds);
        s += ",\"leaves\":[";
        for (size_t l = 0; l < k.leaves.size(); ++l) {
            const Leaf& L = k.leaves[l];
            s += (l ? "," : "") + std::string("{\"loc\":") + json_loc(L.loc) + ",\"dtype\":\"" + dtype_name(L.dtype) +
                 "\",\"zero\":" + (L.zero ? "true" : "false") + ",\"view\":" + json_view(L.v) + "}";
        }
        s += "],\"stores\":[";
        for (size_t l = 0; l < k.stores.size(); ++l) {
            const Store& st = k.stores[l];
            s += (l ? "," : "") + std::string("{\"loc\":") + json_loc(st.loc) + ",\"dtype\":\"" +
                 dtype_name(st.dtype) + "\",\"node\":" + std::to_string(st.node) + ",\"ex\":" + std::to_string(st.ex) +
                 ",\"view\":" + json_view(st.v) + "}";
        }
        s += "],\"ops\":[";
        for (size_t e = 0; e < k.ex.size(); ++e) {
            const Ex& x = k.ex[e];
            const char* nm = x.op == EX_MFMA_ACC ? "MFMA_ACC" : op_name(x.op);
            s += fmt("%s{\"op\":\"%s\",\"dtype\":\"%s\",\"a\":%d,\"b\":%d,\"c\":%d,\"leaf\":%d,\"node\":%d,"
                     "\"cval\":\"%.17g\"",
                     e ? "," : "", x.op == RV_BUFFER ? "LOAD" : nm, dtype_name(x.dtype), x.a, x.b, x.c, x.leaf, x.node,
                     x.cval);
            if (x.op == RV_GATHER)
                s += fmt(",\"gather\":{\"stride\":%lld,\"lo\":%lld,\"hi\":%lld}", (long long)x.g_stride,
                         (long long)x.g_lo, (long long)x.g_hi);
            s += "}";
        }
        s += "]";
        if (k.cls == KClass::SCATTER) {
            s += ",\"scatter\":{\"index\":" + std::to_string(k.sc_index) + ",\"values\":" +
                 std::to_string(k.sc_values) + ",\"base\":" + std::to_string(k.sc_base) +
                 ",\"out\":" + json_loc(k.sc_out) + ",\"out_shape\":[";
            for (size_t d = 0; d < k.sc_out_shape.size(); ++d)
                s += (d ? "," : "") + std::to_string(k.sc_out_shape[d]);
            s += "],\"dtype\":\"" + std::string(dtype_name(k.sc_dtype)) + "\"}";
        }
        s += "}";
    }
    return s + "]}";
}

}  // namespace rv
