// Device-side building blocks of the reduce_view kernels for gfx950 (CDNA4,
// wave64). This text is compiled at run time by the HIP runtime compiler
// together with the kernels the library generates for each graph; it holds
// the parts that do not depend on the graph: dtype conversions, the
// NaN-propagating max, wave reductions, aligned vector access, and the bf16
// MFMA contraction skeleton whose epilogue the generated code supplies.

// ---------------------------------------------------------------------------
// dtype helpers (limn README, "The op set": half widths are widened to
// float32 to compute and rounded back once per result)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float rv_bf2f(unsigned short b) { return __uint_as_float(((unsigned)b) << 16); }

// float32 -> bfloat16, round to nearest even; NaN stays a (quiet) NaN.
// gfx950 converts in one instruction (v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned short rv_f2bf(float f) { return __builtin_bit_cast(unsigned short, (__bf16)f); }

__device__ __forceinline__ float rv_rbf(float x) { return rv_bf2f(rv_f2bf(x)); }
__device__ __forceinline__ float rv_rhf(float x) { return (float)(_Float16)x; }

// MAX with NaN propagation (a NaN anywhere makes the result NaN).
// MAX: a NaN wins, and -0 orders below +0, so a fold gives the same bits in
// any order
__device__ __forceinline__ float rv_maxf(float a, float b) {
    return (a != a) ? a : ((b != b) ? b : (a > b ? a : (b > a ? b : (__builtin_signbit(a) ? b : a))));
}
__device__ __forceinline__ double rv_maxd(double a, double b) {
    return (a != a) ? a : ((b != b) ? b : (a > b ? a : (b > a ? b : (__builtin_signbit(a) ? b : a))));
}

// ---------------------------------------------------------------------------
// aligned vector access: a pack of N elements read or written as one
// 4/8/16-byte memory instruction
// ---------------------------------------------------------------------------
template <class T, int N>
struct __attribute__((aligned(sizeof(T) * N))) rv_pack {
    T v[N];
};

template <class T, int N>
__device__ __forceinline__ rv_pack<T, N> rv_ldv(const T* p) {
    return *reinterpret_cast<const rv_pack<T, N>*>(p);
}

template <class T, int N>
__device__ __forceinline__ void rv_stv(T* p, const rv_pack<T, N>& x) {
    *reinterpret_cast<rv_pack<T, N>*>(p) = x;
}

// Streaming variants: the nontemporal hint for data touched exactly once, so
// it does not evict reused lines (weights, broadcast rows) from the caches.
template <int B>
struct rv_words;
template <>
struct rv_words<4> {
    typedef unsigned type;
};
template <>
struct rv_words<8> {
    typedef __attribute__((ext_vector_type(2))) unsigned type;
};
template <>
struct rv_words<16> {
    typedef __attribute__((ext_vector_type(4))) unsigned type;
};
template <>
struct rv_words<32> {  // 4 doubles: two 16-byte accesses
    typedef __attribute__((ext_vector_type(8))) unsigned type;
};
// a wide operand beside a narrow output (16 floats or doubles feeding 16
// int8 cells): four or eight 16-byte accesses
template <>
struct rv_words<64> {
    typedef __attribute__((ext_vector_type(16))) unsigned type;
};
template <>
struct rv_words<128> {
    typedef __attribute__((ext_vector_type(32))) unsigned type;
};

template <class T, int N>
__device__ __forceinline__ rv_pack<T, N> rv_ldv_nt(const T* p) {
    typedef typename rv_words<sizeof(T) * N>::type W;
    const W w = __builtin_nontemporal_load(reinterpret_cast<const W*>(p));
    rv_pack<T, N> r;
    __builtin_memcpy(&r, &w, sizeof r);
    return r;
}

template <class T, int N>
__device__ __forceinline__ void rv_stv_nt(T* p, const rv_pack<T, N>& x) {
    typedef typename rv_words<sizeof(T) * N>::type W;
    W w;
    __builtin_memcpy(&w, &x, sizeof w);
    __builtin_nontemporal_store(w, reinterpret_cast<W*>(p));
}

// ---------------------------------------------------------------------------
// reductions across the lanes of a row group. A butterfly over xor offsets
// leaves the same bits in every lane of the group: at each level lanes l and
// l^o add the same two values, and IEEE addition is commutative.
// ---------------------------------------------------------------------------
template <int W>
__device__ __forceinline__ float rv_group_sum(float v) {
#pragma unroll
    for (int o = W / 2; o >= 1; o >>= 1) v = v + __shfl_xor(v, o, 64);
    return v;
}

// Workgroup barrier for exchanges through LDS: this wave's LDS accesses
// complete, then s_barrier; the memory clobber keeps the compiler from moving
// memory accesses across it. Unlike __syncthreads() (whose fence waits for
// every outstanding global access) it leaves global loads in flight, so a
// row prefetched before a reduction is still arriving while the row before
// it is reduced.
__device__ __forceinline__ void rv_lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Merge of two online-softmax states (running maximum m, denominator l
// relative to m): both denominators are rescaled to the larger maximum. The
// expression is symmetric in its two operands, so the lanes of a butterfly
// end with the same bits; a state whose maximum is already the result keeps
// its denominator exactly (no -inf - (-inf) for empty or masked ranges).
__device__ __forceinline__ void rv_online_merge(float& m, float& l, float m2, float l2) {
    const float mn = rv_maxf(m, m2);
    const float a1 = (m == mn) ? 1.0f : expf(m - mn);
    const float a2 = (m2 == mn) ? 1.0f : expf(m2 - mn);
    l = l * a1 + l2 * a2;
    m = mn;
}

template <int W>
__device__ __forceinline__ float rv_group_max(float v) {
#pragma unroll
    for (int o = W / 2; o >= 1; o >>= 1) v = rv_maxf(v, __shfl_xor(v, o, 64));
    return v;
}

// The same over float64 (folded in float64) and over ints (a SUM wraps in an
// unsigned total: int arithmetic is exact modulo 2^32, so any order gives the
// same bits).
template <int W>
__device__ __forceinline__ double rv_group_sum(double v) {
#pragma unroll
    for (int o = W / 2; o >= 1; o >>= 1) v = v + __shfl_xor(v, o, 64);
    return v;
}
template <int W>
__device__ __forceinline__ double rv_group_max(double v) {
#pragma unroll
    for (int o = W / 2; o >= 1; o >>= 1) v = rv_maxd(v, __shfl_xor(v, o, 64));
    return v;
}
template <int W>
__device__ __forceinline__ unsigned rv_group_sum(unsigned v) {
#pragma unroll
    for (int o = W / 2; o >= 1; o >>= 1) v = v + (unsigned)__shfl_xor((int)v, o, 64);
    return v;
}
template <int W>
__device__ __forceinline__ int rv_group_max(int v) {
#pragma unroll
    for (int o = W / 2; o >= 1; o >>= 1) {
        const int u = __shfl_xor(v, o, 64);
        v = u > v ? u : v;
    }
    return v;
}

// ---------------------------------------------------------------------------
// bf16 contraction on MFMA: y[m][n] = sum_k A[m][k] * B[k][n] with a float32
// accumulator (limn README, "Backends": a nest that reads as a matmul gets a
// block per output tile, operands staged through on-chip memory and a patch
// of cells held in registers per thread). A bf16 x bf16 product is exact in
// float32, so the contraction equals SUM_k CAST(A) * CAST(B) up to the order
// of the adds.
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(8))) __bf16 rv_bf16x8;
typedef __attribute__((ext_vector_type(16))) float rv_f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned rv_u32x4;
typedef __attribute__((address_space(3))) void rv_lds_void;
typedef __attribute__((ext_vector_type(4))) short rv_s16x4;

// s_waitcnt vmcnt(N) leaving the LDS/export counters free (gfx9 encoding).
#define RV_WAIT_VM(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (7 << 4) | (15 << 8) | ((((N) >> 4) & 3) << 14))
// Workgroup barrier that does not drain the vector-memory counter (a
// __syncthreads() fence waits for every outstanding copy into LDS): this
// wave's LDS reads finish, then s_barrier; the memory clobber keeps the
// compiler from moving LDS accesses across it. Copies the barrier must cover
// are waited for explicitly with RV_WAIT_VM before it.
#define RV_LDS_BARRIER() rv_lds_barrier()

// One k16 step of a wave's TM x TN tiles of v_mfma_f32_32x32x16_bf16.
template <int TM, int TN>
__device__ __forceinline__ void rv_g5_step(rv_f32x16 (&acc)[TM][TN], const rv_bf16x8 (&af)[TM],
                                           const rv_bf16x8 (&bf)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
}

// ---------------------------------------------------------------------------
// The contraction kernel: a 256 x 256 output tile per workgroup of 4 waves,
// each wave a 128 x 128 patch (4 x 4 tiles of v_mfma_f32_32x32x16_bf16, 256
// float32 accumulators per lane: one wave per SIMD, the accumulators fill the
// accumulation registers). Operands go global -> LDS with
// global_load_lds_dwordx4 (each lane's 16 bytes land at the wave's LDS base
// + 16 * lane), so no VGPRs stage them:
//   - A is staged 64 deep, in rows of 128 bytes (whole lines) per copy; a
//     fragment (8 consecutive k of one row) is one ds_read_b128;
//   - an [n][k] B keeps [row][k] rows of 64 bytes per 32-deep k-tile, the
//     16-byte chunks XOR-swizzled by (row / 4) % 4, so 16 consecutive rows
//     read at one chunk cover all 64 banks; a fragment is one ds_read_b128;
//   - a [k][n] B keeps its [k][n] rows of 512 bytes with chunks XOR-swizzled
//     by 4 * (k % 4); a fragment (8 consecutive k of one column) is two
//     ds_read_b64_tr_b16, the gfx950 transposing LDS read.
// With one wave per SIMD nothing else hides latency, so the wave pipelines
// itself: the copies run several k-tiles ahead in LDS stages, and the
// fragments are double buffered in registers (one set for a k-tile's first
// k16 step, one for its second); each k-tile passes one barrier, after which
// every wave's copies of the stage it waited for have landed and nobody reads
// the stage the next copies overwrite. sched_group_barrier pins LDS reads and
// copies between the MFMAs so they hide under the matrix work.
//
// Extents: M, N (each >= 256) and K are the extents the operand buffers
// hold; Mt <= M and Nt <= N are the output's. With RAGGED, a last tile that
// would run past M (or N) starts at M - 256 instead, so every copy stays
// inside the operands and the loop has no edge cases; its cells below the
// nominal tile start belong to the tile before it and, like cells at or
// beyond Mt (Nt), are left out of the epilogue.
// ---------------------------------------------------------------------------
// Per-lane byte offsets of the fragment reads inside one stage (loop
// invariant; the stage's array base, the 32-row tile i (2048 bytes) and, for a
// [k][n] B, the half (4 k-rows, 2048 bytes) and the k16 step (16 k-rows, 8192
// bytes) are added as constants): a[q] for A at k16 step q, b[j] for B tile j
// ([k][n]: step 0, half 0; [n][k]: b[q] as for A).
struct rv_g5_offs {
    unsigned a[2], b[4];
};

template <bool B_KN>
__device__ __forceinline__ rv_g5_offs rv_g5_lane_offs(int wm, int wn, int lane) {
    rv_g5_offs o;
    const int ra = wm * 128 + (lane & 31), swz = ((lane & 31) >> 2) & 3;
#pragma unroll
    for (int q = 0; q < 2; ++q) o.a[q] = (unsigned)(ra * 64 + (((2 * q + (lane >> 5)) ^ swz) << 4));
    if (B_KN) {
        const int g = lane >> 4, jl = lane & 15;
        const int kr = (g >> 1) * 8 + (jl >> 2);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = wn * 128 + j * 32 + (g & 1) * 16 + (jl & 3) * 4;
            o.b[j] = (unsigned)(2 * (kr * 256 + (((n >> 3) ^ ((kr & 3) * 4)) << 3) + (n & 7)));
        }
    } else {
        const int rb = wn * 128 + (lane & 31);
#pragma unroll
        for (int q = 0; q < 2; ++q) o.b[q] = (unsigned)(rb * 64 + (((2 * q + (lane >> 5)) ^ swz) << 4));
        o.b[2] = o.b[3] = 0;
    }
    return o;
}

// interleaving of one k16 step's 16 MFMAs with its NDS LDS reads and NVM
// copies (mask 0x008 MFMA, 0x100 LDS read, 0x010 vector memory). MODE 1: one
// LDS read and one copy after each MFMA while any remain. MODE 2: the LDS
// reads two per MFMA up front (they feed the next step: landing early keeps
// its first MFMA from waiting), the copies one per MFMA after them.
template <int NDS, int NVM, int MODE = 1>
__device__ __forceinline__ void rv_g5_pin() {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (MODE == 1) {
            if (i < NDS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (i < NVM) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
        } else {
            constexpr int R = (NDS + 1) / 2;  // MFMAs that carry LDS reads
            if (2 * i + 1 < NDS)
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            else if (2 * i < NDS)
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (i >= R && i - R < NVM) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
            if (i == 15)
#pragma unroll
                for (int c = 16 - R; c < NVM; ++c) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
        }
    }
}

// The 256 accumulators fill the accumulation registers exactly; left to
// itself the register allocator moves some of them out through memory on
// every k-tile (to make room where the epilogue reads them). Naming them as
// accumulation-register operands of an empty asm at the end of each k-tile
// keeps every one in place across the loop.
__device__ __forceinline__ void rv_g5_keep(rv_f32x16 (&acc)[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) asm volatile("" : "+a"(acc[i][j]));
}

// ---------------------------------------------------------------------------
// The stages: each of the 3 A stages (32 KB) holds two 32-deep k-tiles of
// A; B keeps its 32-deep k-tiles in 4 stages (16 KB), together the 160 KB of
// LDS. At an even k-tile t a wave copies the A stage of tiles t + 4, t + 5
// (8 copies) and B of tile t + 3 (4); at an odd one only B (4). A rows in an
// A stage are 8 chunks of 16 bytes XOR-swizzled by (row / 2) % 8: a fragment
// read (16 rows at one chunk per quarter wave) covers all 64 banks once.
// Staging A 64 deep takes half the L2 requests for its bytes that 64-byte
// halves would. Requires K a multiple of 64.
// ---------------------------------------------------------------------------
struct rv_g6_offs {
    unsigned a[4];  // [parity of the k-tile within its A stage][k16 step]
};

__device__ __forceinline__ rv_g6_offs rv_g6_lane_offs(int wm, int lane) {
    rv_g6_offs o;
    const int ra = wm * 128 + (lane & 31), swz = (ra >> 1) & 7, h = lane >> 5;
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int q = 0; q < 2; ++q) o.a[2 * p + q] = (unsigned)(ra * 128 + (((4 * p + 2 * q + h) ^ swz) << 4));
    return o;
}

template <bool B_KN, int Q, int P>
__device__ __forceinline__ void rv_g6_frags(rv_bf16x8 (&af)[4], rv_bf16x8 (&bf)[4], const unsigned short* As,
                                            const unsigned short* Bs, const rv_g6_offs& oa, const rv_g5_offs& o) {
    const char* pa = reinterpret_cast<const char*>(As) + oa.a[2 * P + Q];
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const rv_bf16x8*>(pa + i * 4096);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (B_KN) {
            const char* pb = reinterpret_cast<const char*>(Bs) + o.b[j] + Q * 8192;
            rv_s16x4 h[2];
#pragma unroll
            for (int half = 0; half < 2; ++half)
                h[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) rv_s16x4*)(pb + half * 2048));
            typedef __attribute__((ext_vector_type(8))) short s16x8;
            s16x8 v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
            bf[j] = __builtin_bit_cast(rv_bf16x8, v);
        } else {
            bf[j] = *reinterpret_cast<const rv_bf16x8*>(reinterpret_cast<const char*>(Bs) + o.b[Q] + j * 2048);
        }
    }
}

// The copies of one k-tile, numbered in issue order: with A (an even tile)
// 0..7 copy the A stage (8 rows of 128 bytes each, rows 64 wave + 8 i), then
// 8..11 B's k-tile; without, 0..3 B's k-tile. Issues those numbered [C0, C1).
template <bool B_KN, bool WITH_A, int C0, int C1>
__device__ __forceinline__ void rv_g6_copy(unsigned short* As, unsigned short* Bs, const unsigned short* __restrict__ A,
                                           const unsigned short* __restrict__ B, long long a_base, long long lda,
                                           long long b_base, long long ldb, int ka, int kb, int wave,
                                           const unsigned (&va)[2], const unsigned (&vb)[2]) {
    constexpr int NA = WITH_A ? 8 : 0;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        if (i < C0 || i >= C1) continue;
        const int r0 = wave * 64 + i * 8;
        const char* g = reinterpret_cast<const char*>(A + a_base + (long long)r0 * lda + ka);
        __builtin_amdgcn_global_load_lds((const void*)(g + va[i & 1]), (rv_lds_void*)(As + r0 * 64), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (NA + i < C0 || NA + i >= C1) continue;
        if (B_KN) {
            const int kr0 = wave * 8 + i * 2;
            const char* g = reinterpret_cast<const char*>(B + b_base + (long long)(kb + kr0) * ldb);
            __builtin_amdgcn_global_load_lds((const void*)(g + vb[i & 1]), (rv_lds_void*)(Bs + kr0 * 256), 16, 0, 0);
        } else {
            const int r0 = wave * 64 + i * 16;
            const char* g = reinterpret_cast<const char*>(B + b_base + (long long)r0 * ldb + kb);
            __builtin_amdgcn_global_load_lds((const void*)(g + vb[0]), (rv_lds_void*)(Bs + r0 * 32), 16, 0, 0);
        }
    }
}

template <bool B_KN, int MODE, class Epi, int PIN = 1, bool RAGGED = false, int PE = 3, int PO = 1,
          int SPLIT = 1>
__device__ __forceinline__ void rv_gemm_w6_bf16(const unsigned short* __restrict__ A,
                                                const unsigned short* __restrict__ B, long long a_off, long long lda,
                                                long long b_off, long long ldb, int M, int N, int K, const Epi& epi,
                                                float* __restrict__ partials, int Mt = 0, int Nt = 0) {
    __shared__ __attribute__((aligned(1024))) unsigned short a0[256 * 64], a1[256 * 64], a2[256 * 64];
    __shared__ __attribute__((aligned(1024))) unsigned short b0[256 * 32], b1[256 * 32], b2[256 * 32], b3[256 * 32];
    constexpr int NDS = B_KN ? 12 : 8;  // LDS read instructions per k16 step
    // copies per k-tile (even: A stage + B tile, odd: B tile), those issued
    // in its first k16 step, and the vmcnt that leaves only copies issued
    // after the next k-tile's B tile in flight (the tile before, and this
    // tile's first-step copies)
    constexpr int CE = 12, CO = 4;
    static_assert(PE >= 0 && PE <= CE && PO >= 0 && PO <= CO, "copies issued in a tile's first step");
    constexpr int WAIT_E = CO + PE, WAIT_O = CE + PO;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int tiles_m = (M + 255) / 256, tiles_n = (N + 255) / 256;
    const int ntiles = tiles_m * tiles_n;
    int tm, tn;
    {
        // SPLIT k-slices: workgroup b takes tile b / SPLIT (in row-major
        // order) of slice b % SPLIT, whose operand offsets and depth K the
        // caller passes; consecutive workgroups run on different XCDs, so the
        // workgroups on one XCD share their slices' A and B panels
        const int bid = (int)blockIdx.x / SPLIT;
        if (SPLIT == 1 && (ntiles & 7) == 0 && (tiles_m & 3) == 0) {
            const int sb = (bid & 7) * (ntiles >> 3) + (bid >> 3);  // XCD-contiguous
            const int group = sb / (4 * tiles_n), within = sb % (4 * tiles_n);
            tm = group * 4 + (within & 3);
            tn = within >> 2;
        } else {
            tm = bid / tiles_n;
            tn = bid % tiles_n;
        }
    }
    const int mlo = tm * 256, nlo = tn * 256;
    const int m0 = RAGGED ? min(mlo, M - 256) : mlo, n0 = RAGGED ? min(nlo, N - 256) : nlo;
    const long long a_base = a_off + (long long)m0 * lda;
    const long long b_base = B_KN ? b_off + n0 : b_off + (long long)n0 * ldb;
    // lane parts of the copy addresses (bytes): A row lane / 8 of 8, chunk
    // lane % 8 swizzled by (row / 2) % 8 = 4 (instruction parity) + lane / 16
    unsigned va[2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
        va[p] = (unsigned)(2 * ((lane >> 3) * lda + (((lane & 7) ^ (4 * p + (lane >> 4))) << 3)));
    unsigned vb[2];
    if (B_KN) {
#pragma unroll
        for (int p = 0; p < 2; ++p)
            vb[p] = (unsigned)(2 * ((lane >> 5) * ldb + (((lane & 31) ^ ((2 * p + (lane >> 5)) * 4)) << 3)));
    } else {
        vb[0] = vb[1] = (unsigned)(2 * ((lane >> 2) * ldb + (((lane & 3) ^ ((lane >> 4) & 3)) << 3)));
    }
    const rv_g5_offs fo = rv_g5_lane_offs<B_KN>(wm, wn, lane);
    const rv_g6_offs fa = rv_g6_lane_offs(wm, lane);

    rv_f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int KT = K / 32, KD = K / 64;
    // copies past the end reload the last tile into a stage nobody reads,
    // so every k-tile issues its fixed number of copies
#define RV_G6_KA(d) (((d) < KD ? (d) : KD - 1) * 64)
#define RV_G6_KB(t) (((t) < KT ? (t) : KT - 1) * 32)
    // prologue: A stages of tiles 0-1 and 2-3, B tiles 0, 1, 2
    rv_g6_copy<B_KN, true, 0, 8>(a0, b0, A, B, a_base, lda, b_base, ldb, RV_G6_KA(0), 0, wave, va, vb);
    rv_g6_copy<B_KN, false, 0, 4>(a0, b0, A, B, a_base, lda, b_base, ldb, 0, RV_G6_KB(0), wave, va, vb);
    rv_g6_copy<B_KN, true, 0, 8>(a1, b0, A, B, a_base, lda, b_base, ldb, RV_G6_KA(1), 0, wave, va, vb);
    rv_g6_copy<B_KN, false, 0, 4>(a0, b1, A, B, a_base, lda, b_base, ldb, 0, RV_G6_KB(1), wave, va, vb);
    rv_g6_copy<B_KN, false, 0, 4>(a0, b2, A, B, a_base, lda, b_base, ldb, 0, RV_G6_KB(2), wave, va, vb);
    RV_WAIT_VM(16);  // A of tiles 0-1 and B of tile 0 have landed
    RV_LDS_BARRIER();
    rv_bf16x8 xa[4], xb[4], ya[4], yb[4];
    rv_g6_frags<B_KN, 0, 0>(xa, xb, a0, b0, fa, fo);
    // one k-tile: CA/PA/CB its A stage, parity and B stage; NA/PN/NB the next
    // tile's; WA the A stage an even tile copies (tiles t + 4, t + 5), WB the
    // B stage of tile t + 3
#define RV_G6_STEP(EVEN, CA, PA, CB, NA, PN, NB, WA, WB, T)                                               \
    {                                                                                                   \
        const int t_ = (T);                                                                             \
        __builtin_amdgcn_sched_barrier(0);                                                              \
        rv_g6_frags<B_KN, 1, PA>(ya, yb, CA, CB, fa, fo);                                               \
        rv_g6_copy<B_KN, EVEN, 0, (EVEN ? PE : PO)>(WA, WB, A, B, a_base, lda, b_base, ldb,             \
                                                    RV_G6_KA(t_ / 2 + 2), RV_G6_KB(t_ + 3), wave, va, vb); \
        rv_g5_step<4, 4>(acc, xa, xb);                                                                  \
        if (PIN) rv_g5_pin<NDS, (EVEN ? PE : PO), PIN>();                                              \
        __builtin_amdgcn_sched_barrier(0);                                                              \
        RV_WAIT_VM(EVEN ? WAIT_E : WAIT_O);                                                             \
        RV_LDS_BARRIER();                                                                               \
        __builtin_amdgcn_sched_barrier(0);                                                              \
        rv_g6_frags<B_KN, 0, PN>(xa, xb, NA, NB, fa, fo);                                               \
        rv_g6_copy<B_KN, EVEN, (EVEN ? PE : PO), (EVEN ? CE : CO)>(WA, WB, A, B, a_base, lda, b_base, ldb, \
                                                                   RV_G6_KA(t_ / 2 + 2), RV_G6_KB(t_ + 3), wave, \
                                                                   va, vb);                           \
        rv_g5_step<4, 4>(acc, ya, yb);                                                                  \
        if (PIN) rv_g5_pin<NDS, (EVEN ? CE - PE : CO - PO), PIN>();                                    \
        __builtin_amdgcn_sched_barrier(0);                                                              \
        rv_g5_keep(acc);                                                                                \
    }
    // whole rounds of 12 k-tiles (A stages cycle every 6, B every 4), then
    // the remaining KT % 12 (even) in order
    int kt = 0;
    for (; kt + 12 <= KT; kt += 12) {
        RV_G6_STEP(true, a0, 0, b0, a0, 1, b1, a2, b3, kt)
        RV_G6_STEP(false, a0, 1, b1, a1, 0, b2, a2, b0, kt + 1)
        RV_G6_STEP(true, a1, 0, b2, a1, 1, b3, a0, b1, kt + 2)
        RV_G6_STEP(false, a1, 1, b3, a2, 0, b0, a0, b2, kt + 3)
        RV_G6_STEP(true, a2, 0, b0, a2, 1, b1, a1, b3, kt + 4)
        RV_G6_STEP(false, a2, 1, b1, a0, 0, b2, a1, b0, kt + 5)
        RV_G6_STEP(true, a0, 0, b2, a0, 1, b3, a2, b1, kt + 6)
        RV_G6_STEP(false, a0, 1, b3, a1, 0, b0, a2, b2, kt + 7)
        RV_G6_STEP(true, a1, 0, b0, a1, 1, b1, a0, b3, kt + 8)
        RV_G6_STEP(false, a1, 1, b1, a2, 0, b2, a0, b0, kt + 9)
        RV_G6_STEP(true, a2, 0, b2, a2, 1, b3, a1, b1, kt + 10)
        RV_G6_STEP(false, a2, 1, b3, a0, 0, b0, a1, b2, kt + 11)
    }
    if (kt < KT) {
        RV_G6_STEP(true, a0, 0, b0, a0, 1, b1, a2, b3, kt)
        RV_G6_STEP(false, a0, 1, b1, a1, 0, b2, a2, b0, kt + 1)
        if (kt + 2 < KT) {
            RV_G6_STEP(true, a1, 0, b2, a1, 1, b3, a0, b1, kt + 2)
            RV_G6_STEP(false, a1, 1, b3, a2, 0, b0, a0, b2, kt + 3)
            if (kt + 4 < KT) {
                RV_G6_STEP(true, a2, 0, b0, a2, 1, b1, a1, b3, kt + 4)
                RV_G6_STEP(false, a2, 1, b1, a0, 0, b2, a1, b0, kt + 5)
                if (kt + 6 < KT) {
                    RV_G6_STEP(true, a0, 0, b2, a0, 1, b3, a2, b1, kt + 6)
                    RV_G6_STEP(false, a0, 1, b3, a1, 0, b0, a2, b2, kt + 7)
                    if (kt + 8 < KT) {
                        RV_G6_STEP(true, a1, 0, b0, a1, 1, b1, a0, b3, kt + 8)
                        RV_G6_STEP(false, a1, 1, b1, a2, 0, b2, a0, b0, kt + 9)
                    }
                }
            }
        }
    }
#undef RV_G6_STEP
#undef RV_G6_KA
#undef RV_G6_KB
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    float* lds_red = reinterpret_cast<float*>(a0);

    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("" : "+a"(acc[i][j]));
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 128 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                const int n = n0 + wn * 128 + j * 32 + (lane & 31);
                if (RAGGED && !(m >= mlo && m < Mt && n >= nlo && n < Nt)) continue;
                const float v = epi(acc[i][j][r], m, n);
                if (MODE == 0)
                    epi.store(m, n, v);
                else
                    part = part + v;
            }
        }
    if (MODE == 1) {
        part = rv_group_sum<64>(part);
        if (lane == 0) lds_red[wave] = part;
        __syncthreads();
        if (tid == 0) partials[blockIdx.x] = ((lds_red[0] + lds_red[1]) + lds_red[2]) + lds_red[3];
    }
}

// ---------------------------------------------------------------------------
// A contraction split over k: the workgroups of slice s store their float32
// accumulators at [s][m][n] (rv_slice_epi, the raw epilogue; planes `plane`
// floats apart, a multiple of 4), and rv_gemm_slices sums the S slices of
// every output cell in slice order, then evaluates the epilogue: stored
// (MODE 0) or summed per workgroup into partials[blockIdx.x] (MODE 1: a
// lane's 4 cells in order, a butterfly over the wave, the 4 waves in order).
// 256 lanes, 4 consecutive cells a lane.
// ---------------------------------------------------------------------------
struct rv_slice_epi {
    float* ws;
    int ld;
    __device__ __forceinline__ float operator()(float acc, int, int) const { return acc; }
    __device__ __forceinline__ void store(int m, int n, float v) const { ws[(long long)m * ld + n] = v; }
};

template <int MODE, class Epi>
__device__ __forceinline__ void rv_gemm_slices(const float* __restrict__ ws, int S, long long plane, int Mt, int Nt,
                                               const Epi& epi, float* __restrict__ partials) {
    __shared__ float lds_red[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const long long cells = (long long)Mt * Nt;
    const long long c0 = ((long long)blockIdx.x * 256 + tid) * 4;
    float y[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (c0 + 4 <= cells) {
        rv_pack<float, 4> v = rv_ldv<float, 4>(ws + c0);
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = v.v[j];
        for (int s = 1; s < S; ++s) {
            v = rv_ldv<float, 4>(ws + s * plane + c0);
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] = y[j] + v.v[j];
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (c0 + j < cells) {
                y[j] = ws[c0 + j];
                for (int s = 1; s < S; ++s) y[j] = y[j] + ws[s * plane + c0 + j];
            }
    }
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (c0 + j >= cells) break;
        const int m = (int)((c0 + j) / Nt), n = (int)((c0 + j) % Nt);
        const float v = epi(y[j], m, n);
        if (MODE == 0)
            epi.store(m, n, v);
        else
            part = part + v;
    }
    if (MODE == 1) {
        part = rv_group_sum<64>(part);
        if (lane == 0) lds_red[wave] = part;
        __syncthreads();
        if (tid == 0) partials[blockIdx.x] = ((lds_red[0] + lds_red[1]) + lds_red[2]) + lds_red[3];
    }
}

// ---------------------------------------------------------------------------
// Fused attention forward, the CUSTOM sdpa_fwd kernel (limn README, "The op
// set": the one CUSTOM kernel, saving the row's logsumexp beside the output;
// Tiki README, "Write the attention kernel at the algorithm level": a
// running maximum m, denominator l and output accumulator per query row,
// updated tile of keys by tile of keys).
//
// The scores are formed transposed, S^T = K Q^T on v_mfma_f32_32x32x16_bf16,
// so a lane of the 32 x 32 result holds 16 scores of ONE query (its column):
// a query's max and sum need one exchange with lane ^ 32 (v_permlane32_swap),
// and rescaling the output accumulator (also transposed, O^T += V^T P^T) is a
// scalar per lane. The probabilities never leave registers: rounded to
// bfloat16 they are the B operand of the second product as they stand. The
// key order the result layout leaves in a lane (keys 4 h .. 4 h + 3 and
// 8 + 4 h .. of each 16, h = lane / 32) is matched by reading V^T from LDS in
// that order. Scores are carried in base 2 (s * scale * log2 e), and each
// exponential is v_exp_f32 of one fma against the reference m.
//
// The reference m is not the running maximum: the probabilities of a tile
// are taken against the m in hand, and only when a query's sum over the tile
// passes 2^8 (or is not finite) does the wave find that tile's maximum, move
// m there, rescale (l, accumulator) and take the tile again; a wave's first
// tile (m = -inf) takes that path directly, so m starts at a maximum and
// later scores far below it fall away as they would against the running
// one. Every probability stays below 2^8, which float32 sums and the bf16
// operand carry with the same relative rounding, and O / l and m + log2 l do
// not depend on which m was used; the per-tile maximum is gone from the
// common path, whose vector work per score is one fma, one exponential, one
// add and half a conversion.
//
// Workgroup: 4 waves, 32 queries each (128 per workgroup). K and V tiles of
// 64 keys go global -> LDS with global_load_lds_dwordx4 (no VGPR staging, no
// LDS stores), NS stages deep, the copies of a tile spread over the 4 waves
// (each copy moves 1 KB: 512 / D key rows). A key row's 16-byte chunks are
// XOR-swizzled (rv_attn_swz): a K fragment read (16 rows at one chunk per
// quarter wave) and a transposing V read (4 rows x 4 chunks per half wave)
// each cover the 64 banks once. Rows past Tk are copies of row Tk - 1, their
// scores masked to -inf. With CAUSAL, key j is hidden from query i when
// j > i: a workgroup stops at the tile holding its last query, a wave skips
// tiles past its queries, and the workgroups with the most keys start first.
// Long rows are split into key chunks over workgroups (wmap); a chunk writes
// its (m, l) and unnormalised accumulator, and rv_attn_merge_chunks folds
// them in chunk order.
// ---------------------------------------------------------------------------
// max and sum over the lane pair (l, l ^ 32) with v_permlane32_swap (no LDS
// round trip): swapped with itself, the pair of results is (lower half's
// value, upper half's value) in every lane, so both lanes compute the same
// expression and get the same bits.
__device__ __forceinline__ float rv_pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float rv_pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void rv_attn_merge(float& m, float& l, float m2, float l2, float& a1, float& a2) {
    const float mn = fmaxf(m, m2);
    a1 = (m == mn) ? 1.0f : __builtin_amdgcn_exp2f(m - mn);
    a2 = (m2 == mn) ? 1.0f : __builtin_amdgcn_exp2f(m2 - mn);
    l = l * a1 + l2 * a2;
    m = mn;
}

// XOR swizzle of key row r's 16-byte chunks in a tile (D / 8 chunks a row,
// rows 2 D bytes apart): chunk c sits at slot c ^ rv_attn_swz<D>(r). A bit
// permutation of the row's position within its 256-byte line run, chosen so
// that rows sharing banks take disjoint chunk slots for both read patterns.
template <int D>
__device__ __forceinline__ int rv_attn_swz(int r) {
    if (D == 32) return (r >> 2) & 3;
    if (D == 64) {
        const int x = (r >> 1) & 7;
        return ((x & 1) << 2) | (x & 2) | (x >> 2);
    }
    const int x = r & 15;
    return ((x & 3) << 2) | (x >> 2);
}

template <int D, bool CAUSAL, bool OUT_BF16, int NS>
__device__ __forceinline__ void rv_attn_fwd_bf16(const unsigned short* __restrict__ Q,
                                                 const unsigned short* __restrict__ K,
                                                 const unsigned short* __restrict__ V, void* __restrict__ O,
                                                 float* __restrict__ L, int Tq, int Tk, float sl2,
                                                 const unsigned* __restrict__ wmap = nullptr, int CK = 0,
                                                 float* __restrict__ opart = nullptr,
                                                 float* __restrict__ mlpart = nullptr, int CMAX = 1) {
    static_assert(D == 32 || D == 64 || D == 128, "head width");
    static_assert(NS >= 2 && NS <= 4, "stages");
    constexpr int TB = 64 * D * 2;  // bytes of one 64-key K (or V) tile
    constexpr int CPW = D / 32;     // copies of each of K and V per wave per tile
    constexpr int CPR = D / 8;      // 16-byte chunks per key row
    // one array per stage: the compiler tells the copies into one stage from
    // reads of another only by the array they address (a read of an array
    // with copies in flight waits for all of them)
    __shared__ __attribute__((aligned(1024))) unsigned char s0[2 * TB], s1[2 * TB];
    __shared__ __attribute__((aligned(1024))) unsigned char s2[NS > 2 ? 2 * TB : 16], s3[NS > 3 ? 2 * TB : 16];
    // the wave index in a scalar register: the per-wave bounds below are
    // scalar branches, with no divergent control flow around the MFMAs
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ql = lane & 31, hh = lane >> 5;
    // which query block and which chunk of its keys: from the map when the
    // keys are split over workgroups (longest blocks first), else one
    // workgroup per block, the longest (under CAUSAL, the last) first
    int jb, ch = 0;
    if (wmap != nullptr) {
        const unsigned e = wmap[blockIdx.x];
        jb = (int)(e >> 16);
        ch = (int)(e & 0xffffu);
    } else {
        jb = CAUSAL ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x;
    }
    const int qb = jb * 128;
    const int q0 = qb + wave * 32;
    const int qi = q0 + ql;
    const long long qbase = (long long)blockIdx.y * Tq;
    const long long kbase = (long long)blockIdx.y * Tk;
    const float ninf = -__builtin_inff();

    int kend = Tk;
    if (CAUSAL) kend = min(Tk, min(Tq, qb + 128));
    // this workgroup's keys: [k0, k1), nt tiles of 64
    const int nchunks = wmap != nullptr ? (kend + CK - 1) / CK : 1;
    const int k0 = wmap != nullptr ? ch * CK : 0;
    const int k1 = wmap != nullptr ? min(kend, k0 + CK) : kend;
    const int nt = (k1 - k0 + 63) / 64;

    // copy i of this wave (copy j = wave + 4 i of the tile, 1 KB of LDS at
    // 1024 j): its lane's key row within the tile and global byte column
    int crow[CPW], ccol[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        const int n = 64 * (wave + 4 * i) + lane, r = n / CPR;
        crow[i] = r;
        ccol[i] = 16 * ((n % CPR) ^ rv_attn_swz<D>(r));
    }
    auto issue = [&](unsigned char* ks, int t) {  // the copies of tile t into stage ks
        const int kt0 = k0 + 64 * t;
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
            const long long row = kbase + min(kt0 + crow[i], Tk - 1);
            const char* gk = reinterpret_cast<const char*>(K) + row * (2 * D) + ccol[i];
            const char* gv = reinterpret_cast<const char*>(V) + row * (2 * D) + ccol[i];
            __builtin_amdgcn_global_load_lds((const void*)gk, (rv_lds_void*)(ks + 1024 * (wave + 4 * i)), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const void*)gv, (rv_lds_void*)(ks + TB + 1024 * (wave + 4 * i)), 16, 0,
                                             0);
        }
    };
    // Loads are unconditional, with rows clamped into range: a query row
    // past Tq computes on row Tq - 1 and is never stored. q is
    // loaded before the first copies: the loop's first wait covers it.
    rv_bf16x8 qf[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        rv_u32x4 w = *reinterpret_cast<const rv_u32x4*>(Q + (qbase + min(qi, Tq - 1)) * D + 16 * s + 8 * hh);
        qf[s] = __builtin_bit_cast(rv_bf16x8, w);
    }

    issue(s0, 0);
    if (NS > 2) issue(s1, min(1, nt - 1));
    if (NS > 3) issue(s2, min(2, nt - 1));

    // fragment offsets within a stage: K (row ql of a 32-key half, chunk
    // 2 s + hh; the half adds 64 D bytes) and the two transposing V reads
    // of head-dim tile dt (rows 4 (g / 2) + j / 4 (+ 8) of each 16 keys,
    // 4 dims at 16 (g % 2) + 4 (j % 4); the 16-key step adds 32 D bytes)
    unsigned koff[D / 16], voff[D / 32][2];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) koff[s] = (unsigned)(ql * 2 * D + 16 * ((2 * s + hh) ^ rv_attn_swz<D>(ql)));
    {
        const int g = lane >> 4, j = lane & 15;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int row = 4 * (g >> 1) + (j >> 2) + 8 * h;
                const int col = dt * 32 + (g & 1) * 16 + (j & 3) * 4;
                voff[dt][h] = (unsigned)(TB + row * 2 * D + 16 * ((col >> 3) ^ rv_attn_swz<D>(row)) + (col & 7) * 2);
            }
    }

    rv_f32x16 oacc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.0f;
    float m = ninf, l = 0.0f;

    // S^T for the 64 keys of tile t (stage st) as two 32 x 32 tiles (A = K
    // rows: lane = key ql of the half, head dims 16 s + 8 hh ..; B = Q^T),
    // hidden keys set to -inf
    auto scores = [&](const unsigned char* st, int kb, float (&sv)[32]) {
        rv_f32x16 sacc[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[u][r] = 0.0f;
#pragma unroll
            for (int s = 0; s < D / 16; ++s) {
                const rv_bf16x8 af = *reinterpret_cast<const rv_bf16x8*>(st + koff[s] + u * 64 * D);
                sacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[s], sacc[u], 0, 0, 0);
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) sv[16 * u + r] = sacc[u][r];
        if (kb + 64 > k1 || (CAUSAL && kb + 63 > q0)) {  // wave-uniform
#pragma unroll
            for (int r = 0; r < 32; ++r) {
                const int key = kb + (r >> 4) * 32 + ((r & 15) >> 2) * 8 + hh * 4 + (r & 3);
                if (key >= k1 || (CAUSAL && key > qi)) sv[r] = ninf;
            }
        }
    };
    // probabilities of the scores against m, and their sum over the
    // query's 64 keys (four interleaved partial sums, then a tree: four
    // short dependency chains instead of one of 32 adds); while every key
    // seen is hidden (m = -inf) every score is -inf and exp2(-inf - 0) = 0
    auto probs = [&](const float (&sv)[32], float (&pr)[32]) {
        const float mns = m == ninf ? 0.0f : m;
        float ps[4];
#pragma unroll
        for (int r = 0; r < 32; ++r) {
            pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r], sl2, -mns));
            ps[r & 3] = r < 4 ? pr[r] : ps[r & 3] + pr[r];
        }
        return rv_pair_sum((ps[0] + ps[1]) + (ps[2] + ps[3]));
    };
    // one tile: cur its stage, nxt the stage of tile t + NS - 1
    auto step = [&](const unsigned char* cur, unsigned char* nxt, int t) {
        // tile t has landed for this wave (the NS - 2 after it may still
        // fly), then for every wave; after the barrier nobody reads tile
        // t - 1's stage, which the copies of tile t + NS - 1 overwrite. Past
        // the last tile the copies repeat it into stages nobody reads again:
        // with no branch around them, every copy names its stage's array
        // (copies under a branch get merged across stages, and a read of any
        // stage then waits for all of them).
        RV_WAIT_VM(2 * CPW * (NS - 2));
        RV_LDS_BARRIER();
        issue(nxt, min(t + NS - 1, nt - 1));
        const int kb = k0 + 64 * t;
        // keys all hidden from this wave's queries (wave-uniform)
        if (CAUSAL && kb > q0 + 31) return;
        float pr[32];
        float ps = 0.0f;
        // the first tile a wave takes (m still -inf; it holds a key every
        // query of the wave sees) goes straight to the exact path
        bool over = m == ninf;
        bool slow = __builtin_amdgcn_ballot_w64(over) != 0;
        if (!slow) {
            float sv[32];
            scores(cur, kb, sv);
            ps = probs(sv, pr);
            over = !(ps <= 256.0f);
            slow = __builtin_amdgcn_ballot_w64(over) != 0;
        }
        if (slow) {  // wave-uniform, rare
            // the scores again (cheaper than holding them), the tile's
            // maximum, the rescale, the probabilities against the new m
            float sv[32];
            scores(cur, kb, sv);
            float cm = sv[0];
#pragma unroll
            for (int r = 1; r < 32; ++r) cm = fmaxf(cm, sv[r]);
            // max(s) * c equals max(s * c) for c > 0 (rounding is monotonic);
            // a sum past 2^8 has a probability past 4, so cm2 > m there
            const float cm2 = rv_pair_max(cm) * sl2;
            const bool grow = over && cm2 > m;
            const float mn = grow ? cm2 : m;
            const float alpha = grow ? __builtin_amdgcn_exp2f(m - mn) : 1.0f;  // exp2(-inf) = 0
            l = l * alpha;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
            m = mn;
            ps = probs(sv, pr);
        }
        l = l + ps;
        // O^T += V^T P^T over the 64 keys (four k16 steps); P to bf16 two
        // at a time (one v_cvt_pk_bf16_f32 per pair)
        rv_bf16x8 pb[4];
        typedef __attribute__((ext_vector_type(2))) float f32x2;
        typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x2 f = {pr[8 * s + 2 * i], pr[8 * s + 2 * i + 1]};
                const bf16x2 h = __builtin_convertvector(f, bf16x2);
                pb[s][2 * i] = h[0];
                pb[s][2 * i + 1] = h[1];
            }
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                // k16 step s: keys 16 s + 4 hh + 0..3 and + 8, two
                // transposing reads of the key-major V tile
                typedef __attribute__((address_space(3))) rv_s16x4 lds_s16x4;
                typedef __attribute__((address_space(3))) unsigned char lds_u8;
                const lds_u8* vb = (const lds_u8*)(cur + s * 32 * D);
                const rv_s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + voff[dt][0]));
                const rv_s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + voff[dt][1]));
                typedef __attribute__((ext_vector_type(8))) short s16x8;
                const s16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(rv_bf16x8, a8), pb[s], oacc[dt],
                                                                   0, 0, 0);
            }
    };
    // the stages cycle every NS tiles: unrolled so that every LDS access
    // names its stage's array
    int t = 0;
    if (NS == 2) {
        for (; t + 2 <= nt; t += 2) {
            step(s0, s1, t);
            step(s1, s0, t + 1);
        }
        if (t < nt) step(s0, s1, t);
    } else if (NS == 3) {
        for (; t + 3 <= nt; t += 3) {
            step(s0, s2, t);
            step(s1, s0, t + 1);
            step(s2, s1, t + 2);
        }
        if (t < nt) {
            step(s0, s2, t);
            if (t + 1 < nt) step(s1, s0, t + 1);
        }
    } else {
        for (; t + 4 <= nt; t += 4) {
            step(s0, s3, t);
            step(s1, s0, t + 1);
            step(s2, s1, t + 2);
            step(s3, s2, t + 3);
        }
        if (t < nt) {
            step(s0, s3, t);
            if (t + 1 < nt) {
                step(s1, s0, t + 1);
                if (t + 2 < nt) step(s2, s1, t + 2);
            }
        }
    }
    // no copy into LDS outlives the workgroup
    RV_WAIT_VM(0);
    if (qi < Tq && nchunks > 1) {  // a partial: (m, l) and the unnormalised accumulator
        const long long slot = ((long long)blockIdx.y * ((Tq + 127) / 128) + jb) * CMAX + ch;
        float* op = opart + (slot * 128 + (qi - qb)) * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                rv_pack<float, 4> pk;
#pragma unroll
                for (int i = 0; i < 4; ++i) pk.v[i] = oacc[dt][4 * g + i];
                rv_stv<float, 4>(op + dt * 32 + g * 8 + hh * 4, pk);
            }
        if (hh == 0) {
            mlpart[(slot * 128 + (qi - qb)) * 2] = m;
            mlpart[(slot * 128 + (qi - qb)) * 2 + 1] = l;
        }
        return;
    }
    if (qi < Tq) {
        const float inv = 1.0f / l;
        if (O != nullptr) {
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const long long at = (qbase + qi) * D + dt * 32 + g * 8 + hh * 4;
                    if (OUT_BF16) {
                        rv_pack<unsigned short, 4> pk;
#pragma unroll
                        for (int i = 0; i < 4; ++i) pk.v[i] = rv_f2bf(oacc[dt][4 * g + i] * inv);
                        rv_stv<unsigned short, 4>(reinterpret_cast<unsigned short*>(O) + at, pk);
                    } else {
                        rv_pack<float, 4> pk;
#pragma unroll
                        for (int i = 0; i < 4; ++i) pk.v[i] = oacc[dt][4 * g + i] * inv;
                        rv_stv<float, 4>(reinterpret_cast<float*>(O) + at, pk);
                    }
                }
        }
        if (L != nullptr && hh == 0) L[qbase + qi] = m * 0.693147180559945309f + logf(l);
    }
}

// Merge of the key chunks of a query block: D / 4 lanes per query, each
// folding 4 accumulator columns (and the query's (m, l)) over the chunks in
// chunk order, as the key groups of one workgroup are folded, then
// O = acc / l and L = m ln 2 + log l. Grid: (query blocks x 128 / QPB, heads)
// with QPB = 256 / (D / 4) queries per workgroup. Blocks with one chunk were
// written whole by the forward kernel.
template <int D, bool CAUSAL, bool OUT_BF16>
__device__ __forceinline__ void rv_attn_merge_chunks(void* __restrict__ O, float* __restrict__ L,
                                                     const float* __restrict__ opart,
                                                     const float* __restrict__ mlpart, int Tq, int Tk, int CK,
                                                     int CMAX) {
    constexpr int TQ = D / 4, QPB = 256 / TQ;
    const int sub = (int)blockIdx.x % (128 / QPB), jb = (int)blockIdx.x / (128 / QPB);
    const int ql = sub * QPB + (int)threadIdx.x / TQ, d0 = ((int)threadIdx.x % TQ) * 4;
    const int qb = jb * 128, qi = qb + ql;
    const int kend = CAUSAL ? min(Tk, min(Tq, qb + 128)) : Tk;
    const int nchunks = (kend + CK - 1) / CK;
    if (nchunks <= 1 || qi >= Tq) return;
    const long long slot0 = ((long long)blockIdx.y * ((Tq + 127) / 128) + jb) * CMAX;
    float m = mlpart[(slot0 * 128 + ql) * 2], l = mlpart[(slot0 * 128 + ql) * 2 + 1];
    rv_pack<float, 4> acc = rv_ldv<float, 4>(opart + (slot0 * 128 + ql) * D + d0);
#pragma unroll 4
    for (int c = 1; c < nchunks; ++c) {
        const long long sl = (slot0 + c) * 128 + ql;
        const rv_pack<float, 4> v = rv_ldv<float, 4>(opart + sl * D + d0);
        float a1, a2;
        rv_attn_merge(m, l, mlpart[sl * 2], mlpart[sl * 2 + 1], a1, a2);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc.v[i] = acc.v[i] * a1 + v.v[i] * a2;
    }
    const float inv = 1.0f / l;
    const long long at = ((long long)blockIdx.y * Tq + qi) * D + d0;
    if (O != nullptr) {
        if (OUT_BF16) {
            rv_pack<unsigned short, 4> pk;
#pragma unroll
            for (int i = 0; i < 4; ++i) pk.v[i] = rv_f2bf(acc.v[i] * inv);
            rv_stv<unsigned short, 4>(reinterpret_cast<unsigned short*>(O) + at, pk);
        } else {
            rv_pack<float, 4> pk;
#pragma unroll
            for (int i = 0; i < 4; ++i) pk.v[i] = acc.v[i] * inv;
            rv_stv<float, 4>(reinterpret_cast<float*>(O) + at, pk);
        }
    }
    if (L != nullptr && d0 == 0) L[(long long)blockIdx.y * Tq + qi] = m * 0.693147180559945309f + logf(l);
}

// Deterministic fold of `count` float partials into one value: each thread
// adds a strided subset in ascending order, then a fixed binary tree in LDS.
// No atomics, so two runs give the same bits.
__device__ __forceinline__ float rv_fold_sum(const float* __restrict__ part, long long count) {
    __shared__ float s[256];
    const int t = threadIdx.x;
    float acc = 0.0f;
    for (long long i = t; i < count; i += 256) acc = acc + part[i];
    s[t] = acc;
    __syncthreads();
#pragma unroll
    for (int w = 128; w > 0; w >>= 1) {
        if (t < w) s[t] = s[t] + s[t + w];
        __syncthreads();
    }
    return s[0];
}

// ---------------------------------------------------------------------------
// Scatter-add helpers.
//
// Stable LSD radix sort of (key, value) u32 pairs with 8-bit digits, in
// tiles of 2048 pairs (256 lanes, 8 rounds of 256 consecutive pairs). Per
// pass: digit counts per tile, an exclusive scan of each digit's tile
// counts, and a move that places every pair at
//   (pairs of smaller digits) + (pairs of its digit in earlier tiles)
//   + (pairs of its digit earlier in this tile),
// the last from wave ballots, so pairs with equal digits keep their order.
// Counts are integers (LDS atomics only count), so every run places every
// pair at the same position.
// ---------------------------------------------------------------------------
#define RV_RS_TILE 2048

// Exclusive scan of v over the 256 lanes of the workgroup; `tot` gets the
// total. `w` is 4 words of LDS.
__device__ __forceinline__ unsigned rv_scan256(unsigned v, unsigned* w, unsigned& tot) {
    const unsigned lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    unsigned x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const unsigned y = (unsigned)__shfl_up((int)x, o, 64);
        if (lane >= (unsigned)o) x += y;
    }
    if (lane == 63u) w[wave] = x;
    __syncthreads();
    unsigned pre = 0u;
    for (unsigned q = 0; q < wave; ++q) pre += w[q];
    tot = w[0] + w[1] + w[2] + w[3];
    __syncthreads();
    return pre + x - v;
}

// One workgroup per digit (blockIdx.x): counts[d * nb + b] becomes the
// number of pairs of digit d in tiles before b; counts[256 * nb + d] gets the
// digit's total.
__device__ __forceinline__ void rv_rs_scan(unsigned* __restrict__ counts, unsigned nb) {
    __shared__ unsigned w[4];
    unsigned* row = counts + (size_t)blockIdx.x * nb;
    unsigned carry = 0u;
    for (unsigned c0 = 0; c0 < nb; c0 += 256u) {
        const unsigned j = c0 + threadIdx.x;
        const unsigned v = j < nb ? row[j] : 0u;
        unsigned tot;
        const unsigned ex = rv_scan256(v, w, tot);
        if (j < nb) row[j] = carry + ex;
        carry += tot;
    }
    if (threadIdx.x == 0) counts[(size_t)256 * nb + blockIdx.x] = carry;
}

// Digit counts of one tile (one workgroup per tile): counts[d * nb + tile].
__device__ __forceinline__ void rv_rs_hist(const unsigned* __restrict__ keys, unsigned* __restrict__ counts,
                                           long long n, unsigned nb, int shift) {
    __shared__ unsigned h[256];
    const unsigned t = threadIdx.x;
    h[t] = 0u;
    __syncthreads();
    const long long base = (long long)blockIdx.x * RV_RS_TILE;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const long long j = base + r * 256 + t;
        if (j < n) atomicAdd(&h[(keys[j] >> shift) & 255u], 1u);
    }
    __syncthreads();
    counts[(size_t)t * nb + blockIdx.x] = h[t];
}

// Exclusive scan of v over the 1024 lanes of the workgroup (16 waves);
// `tot` gets the total. `w` is 16 words of LDS.
__device__ __forceinline__ unsigned rv_scan1024(unsigned v, unsigned* w, unsigned& tot) {
    const unsigned lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    unsigned x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const unsigned y = (unsigned)__shfl_up((int)x, o, 64);
        if (lane >= (unsigned)o) x += y;
    }
    if (lane == 63u) w[wave] = x;
    __syncthreads();
    unsigned pre = 0u, all = 0u;
    for (unsigned q = 0; q < 16u; ++q) {
        pre += q < wave ? w[q] : 0u;
        all += w[q];
    }
    tot = all;
    __syncthreads();
    return pre + x - v;
}

// The move of one radix pass, 1024 lanes (16 waves) per tile of 2048 pairs
// in 2 rounds. SELF (at most 64 tiles): every workgroup counts the digits
// of every tile in LDS; otherwise `counts` holds the per-tile prefixes and
// digit totals from rv_rs_hist and rv_rs_scan.
// (key, value) pairs of a radix pass: from the previous pass's arrays, or
// (first pass) computed where they are needed from the index by a functor
// f(j, key, value), so no kernel writes them first
struct rv_rs_mem {
    const unsigned* __restrict__ k;
    const unsigned* __restrict__ v;
    __device__ __forceinline__ void get(long long j, unsigned& key, unsigned& val) const {
        key = k[j];
        val = v[j];
    }
};
template <class F>
struct rv_rs_fn {
    F f;
    __device__ __forceinline__ void get(long long j, unsigned& key, unsigned& val) const { f(j, key, val); }
};

template <bool SELF, class KV>
__device__ __forceinline__ void rv_rs_move_kv(const KV& src, unsigned* __restrict__ okeys,
                                              unsigned* __restrict__ ovals, const unsigned* __restrict__ counts,
                                              long long n, unsigned nb, int shift);

template <bool SELF>
__device__ __forceinline__ void rv_rs_move(const unsigned* __restrict__ keys, const unsigned* __restrict__ vals,
                                           unsigned* __restrict__ okeys, unsigned* __restrict__ ovals,
                                           const unsigned* __restrict__ counts, long long n, unsigned nb, int shift) {
    rv_rs_move_kv<SELF>(rv_rs_mem{keys, vals}, okeys, ovals, counts, n, nb, shift);
}

template <bool SELF, class KV>
__device__ __forceinline__ void rv_rs_move_kv(const KV& src, unsigned* __restrict__ okeys,
                                              unsigned* __restrict__ ovals, const unsigned* __restrict__ counts,
                                              long long n, unsigned nb, int shift) {
    __shared__ unsigned run[256];
    __shared__ unsigned wc[16][256];
    __shared__ unsigned w[16];
    const unsigned t = threadIdx.x, lane = t & 63u, wave = t >> 6;
    unsigned total = 0u, pre = 0u;
    if (SELF) {
        __shared__ unsigned hc[256 * 64];
        for (unsigned q = t; q < 256u * nb; q += 1024u) hc[q] = 0u;
        __syncthreads();
        // 32 loads in flight per lane (32768 keys in one round trip); the
        // counts are tile-major, so the 64 lanes of a wave (one tile, random
        // digits) spread over the banks instead of meeting in a few
        for (long long j0 = t; j0 < n; j0 += 1024 * 32) {
            unsigned kv[32];
#pragma unroll
            for (int u = 0; u < 32; ++u) {
                unsigned vv;
                kv[u] = 0u;
                if (j0 + u * 1024 < n) src.get(j0 + u * 1024, kv[u], vv);
            }
#pragma unroll
            for (int u = 0; u < 32; ++u)
                if (j0 + u * 1024 < n)
                    atomicAdd(&hc[(unsigned)((j0 + u * 1024) >> 11) * 256u + ((kv[u] >> shift) & 255u)], 1u);
        }
        __syncthreads();
        if (t < 256u)
            for (unsigned b = 0; b < nb; ++b) {
                const unsigned v = hc[b * 256u + t];
                total += v;
                pre += b < blockIdx.x ? v : 0u;
            }
    } else if (t < 256u) {
        total = counts[(size_t)256 * nb + t];
        pre = counts[(size_t)t * nb + blockIdx.x];
    }
    unsigned tot;
    const unsigned start = rv_scan1024(total, w, tot);
    // lane t < 256 owns digit t: its running position and its column of
    // the per-wave counts (cleared by the owner only, after every reader)
    if (t < 256u) {
        run[t] = start + pre;
#pragma unroll
        for (int q = 0; q < 16; ++q) wc[q][t] = 0u;
    }
    const unsigned long long below = (1ull << lane) - 1ull;
    // both rounds' pairs loaded up front (one round trip instead of two)
    unsigned rk[2], rvv[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const long long j = (long long)blockIdx.x * RV_RS_TILE + r * 1024 + t;
        rk[r] = rvv[r] = 0u;
        if (j < n) src.get(j, rk[r], rvv[r]);
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        __syncthreads();
        const long long j = (long long)blockIdx.x * RV_RS_TILE + r * 1024 + t;
        const bool ok = j < n;
        const unsigned key = rk[r], val = rvv[r];
        const unsigned d = (key >> shift) & 255u;
        unsigned long long same = __builtin_amdgcn_ballot_w64(ok);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const bool bit = (d >> b) & 1u;
            const unsigned long long m = __builtin_amdgcn_ballot_w64(bit);
            same &= bit ? m : ~m;
        }
        const unsigned rank = (unsigned)__popcll(same & below);
        if (ok && rank == 0u) wc[wave][d] = (unsigned)__popcll(same);
        __syncthreads();
        if (ok) {
            unsigned pos = run[d] + rank;
            for (unsigned q = 0; q < wave; ++q) pos += wc[q][d];
            if ((long long)pos < n) {  // always, when the counts match the keys
                okeys[pos] = key;
                ovals[pos] = val;
            }
        }
        __syncthreads();
        if (t < 256u) {
            unsigned add = 0u;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                add += wc[q][t];
                wc[q][t] = 0u;
            }
            run[t] += add;
        }
    }
}

// Unordered scatter-add: hardware atomic adds (device scope, relaxed).
__device__ __forceinline__ void rv_atomic_add(float* p, float v) { unsafeAtomicAdd(p, v); }
__device__ __forceinline__ void rv_atomic_add(double* p, double v) { unsafeAtomicAdd(p, v); }
__device__ __forceinline__ void rv_atomic_add(int* p, int v) { atomicAdd(p, v); }
