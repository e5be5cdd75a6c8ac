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
__device__ __forceinline__ float rv_maxf(float a, float b) {
    return (a != a) ? a : ((b != b) ? b : (a > b ? a : b));
}
__device__ __forceinline__ double rv_maxd(double a, double b) {
    return (a != a) ? a : ((b != b) ? b : (a > b ? a : b));
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

template <int W>
__device__ __forceinline__ float rv_group_max(float v) {
#pragma unroll
    for (int o = W / 2; o >= 1; o >>= 1) v = rv_maxf(v, __shfl_xor(v, o, 64));
    return v;
}

// ---------------------------------------------------------------------------
// bf16 contraction on MFMA: y[m][n] = sum_k A[m][k] * B[k][n] with a float32
// accumulator (limn README, "Backends": a nest that reads as a matmul gets a
// block per output tile, operands staged through on-chip memory and a patch
// of cells held in registers per thread).
//
// Tile 128 x 128 x 64 per workgroup of 4 waves (2 x 2), each wave owning a
// 64 x 64 patch as 2 x 2 tiles of v_mfma_f32_32x32x16_bf16. A is read as
// [m][k] rows; B is staged in LDS as [n][k] so that every lane's MFMA operand
// (8 consecutive k of one row or column) is one 16-byte LDS read. A B stored
// [k][n] is transposed on its way into LDS: each thread loads 4 k-rows of 8
// n and writes 8 n-rows of 4 k. Two LDS stages: the global loads of tile
// k+1 are in flight while tile k is multiplied. Workgroups are remapped so
// that each of the 8 XCDs runs a contiguous block of output tiles (shared
// A rows stay in that XCD's L2).
//
// Product exactness: a bf16 x bf16 product is exact in float32, so the
// contraction equals SUM_k CAST(A) * CAST(B) up to the order of the adds.
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(8))) __bf16 rv_bf16x8;
typedef __attribute__((ext_vector_type(16))) float rv_f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned rv_u32x4;

#define RV_GEMM_BM 128
#define RV_GEMM_BN 128
#define RV_GEMM_BK 64
#define RV_GEMM_LDK 72  // LDS row pitch in bf16 (64 + 8 pad)

template <bool B_KN>
struct rv_gemm_stage {
    rv_u32x4 a[4];
    rv_u32x4 b[4];
};

// Global -> registers for one k-tile.
template <bool B_KN>
__device__ __forceinline__ void rv_gemm_load(rv_gemm_stage<B_KN>& s, const unsigned short* __restrict__ A,
                                             const unsigned short* __restrict__ B, long long a_base, long long lda,
                                             long long b_base, long long ldb, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int v = tid + 256 * i;
        int row = v >> 3, kc = (v & 7) * 8;
        s.a[i] = *reinterpret_cast<const rv_u32x4*>(A + a_base + (long long)row * lda + k0 + kc);
    }
    if (B_KN) {
        int nc = (tid & 15) * 8, kg = (tid >> 4) * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            s.b[j] = *reinterpret_cast<const rv_u32x4*>(B + b_base + (long long)(k0 + kg + j) * ldb + nc);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int v = tid + 256 * i;
            int row = v >> 3, kc = (v & 7) * 8;
            s.b[i] = *reinterpret_cast<const rv_u32x4*>(B + b_base + (long long)row * ldb + k0 + kc);
        }
    }
}

// Registers -> LDS stage (A as [m][k], B as [n][k]).
template <bool B_KN>
__device__ __forceinline__ void rv_gemm_store(const rv_gemm_stage<B_KN>& s, unsigned short* As, unsigned short* Bs,
                                              int tid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int v = tid + 256 * i;
        int row = v >> 3, kc = (v & 7) * 8;
        *reinterpret_cast<rv_u32x4*>(As + row * RV_GEMM_LDK + kc) = s.a[i];
    }
    if (B_KN) {
        int nc = (tid & 15) * 8, kg = (tid >> 4) * 4;
        // s.b[j] holds B[kg + j][nc .. nc + 7]; write column nc + e as the 4
        // consecutive k values (kg .. kg + 3).
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            int w = e >> 1, hi = e & 1;
            unsigned k01, k23;
            unsigned x0 = s.b[0][w], x1 = s.b[1][w], x2 = s.b[2][w], x3 = s.b[3][w];
            if (hi) {
                k01 = (x0 >> 16) | (x1 & 0xffff0000u);
                k23 = (x2 >> 16) | (x3 & 0xffff0000u);
            } else {
                k01 = (x0 & 0xffffu) | (x1 << 16);
                k23 = (x2 & 0xffffu) | (x3 << 16);
            }
            typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
            u32x2 pk;
            pk[0] = k01;
            pk[1] = k23;
            *reinterpret_cast<u32x2*>(Bs + (nc + e) * RV_GEMM_LDK + kg) = pk;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int v = tid + 256 * i;
            int row = v >> 3, kc = (v & 7) * 8;
            *reinterpret_cast<rv_u32x4*>(Bs + row * RV_GEMM_LDK + kc) = s.b[i];
        }
    }
}

// Runs the contraction for the tile of this workgroup and hands every
// (m, n, y) to `epi`, which returns the value the epilogue stores or sums.
// MODE 0: epi.store(m, n, v); MODE 1: per-workgroup sum of v written to
// partials[blockIdx.x].
template <bool B_KN, int MODE, class Epi>
__device__ __forceinline__ void rv_gemm_bf16(const unsigned short* __restrict__ A, const unsigned short* __restrict__ B,
                                             long long a_off, long long lda, long long b_off, long long ldb, int M,
                                             int N, int K, const Epi& epi, float* __restrict__ partials) {
    __shared__ __attribute__((aligned(16))) unsigned short lds_a[2][RV_GEMM_BM * RV_GEMM_LDK];
    __shared__ __attribute__((aligned(16))) unsigned short lds_b[2][RV_GEMM_BN * RV_GEMM_LDK];
    __shared__ float lds_red[4];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tiles_n = N / RV_GEMM_BN;
    const int ntiles = (M / RV_GEMM_BM) * tiles_n;
    int bid = blockIdx.x;
    if ((ntiles & 7) == 0) bid = (bid & 7) * (ntiles >> 3) + (bid >> 3);  // XCD-contiguous tiles
    const int m0 = (bid / tiles_n) * RV_GEMM_BM, n0 = (bid % tiles_n) * RV_GEMM_BN;
    const long long a_base = a_off + (long long)m0 * lda;
    const long long b_base = B_KN ? b_off + n0 : b_off + (long long)n0 * ldb;

    rv_f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    rv_gemm_stage<B_KN> st;
    rv_gemm_load<B_KN>(st, A, B, a_base, lda, b_base, ldb, 0, tid);
    rv_gemm_store<B_KN>(st, lds_a[0], lds_b[0], tid);
    __syncthreads();
    const int KT = K / RV_GEMM_BK;
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) rv_gemm_load<B_KN>(st, A, B, a_base, lda, b_base, ldb, (kt + 1) * RV_GEMM_BK, tid);
        const unsigned short* As = lds_a[cur];
        const unsigned short* Bs = lds_b[cur];
#pragma unroll
        for (int kk = 0; kk < RV_GEMM_BK; kk += 16) {
            rv_bf16x8 af[2], bf[2];
            const int kq = kk + (lane >> 5) * 8;
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *reinterpret_cast<const rv_bf16x8*>(As + (wm * 64 + i * 32 + (lane & 31)) * RV_GEMM_LDK + kq);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bf[j] = *reinterpret_cast<const rv_bf16x8*>(Bs + (wn * 64 + j * 32 + (lane & 31)) * RV_GEMM_LDK + kq);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < KT) rv_gemm_store<B_KN>(st, lds_a[cur ^ 1], lds_b[cur ^ 1], tid);
        __syncthreads();
    }

    // epilogue: lane holds y at rows (r/4)*8 + (lane/32)*4 + r%4, column lane%32
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                const int n = n0 + wn * 64 + j * 32 + (lane & 31);
                const float v = epi(acc[i][j][r], m, n);
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
// The large-tile contraction: 256 x 256 x 64 per workgroup of 4 waves (one per
// SIMD), each wave a 128 x 128 patch as 4 x 4 tiles of
// v_mfma_f32_32x32x16_bf16 (256 float32 accumulators per lane). Per k16 step a
// wave reads 8 operand fragments from LDS for 16 MFMAs, half the LDS traffic
// per MFMA of the 128 x 128 tile. The next k-tile's global loads are issued
// before the current tile's MFMAs and written to the other LDS stage halfway
// through them. A 4096^3 problem is 256 workgroups: one per CU; each XCD gets
// a 4 x 8 block of tiles so its L2 holds the A rows and B columns it shares.
// ---------------------------------------------------------------------------
#define RV_G2_BM 256
#define RV_G2_BN 256
#define RV_G2_BK 64
#define RV_G2_LDK 72

template <bool B_KN>
struct rv_g2_regs {
    rv_u32x4 a[8];
    rv_u32x4 b[8];
};

template <bool B_KN>
__device__ __forceinline__ void rv_g2_load(rv_g2_regs<B_KN>& s, const unsigned short* __restrict__ A,
                                           const unsigned short* __restrict__ B, long long a_base, long long lda,
                                           long long b_base, long long ldb, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int v = tid + 256 * i;
        int row = v >> 3, kc = (v & 7) * 8;
        s.a[i] = *reinterpret_cast<const rv_u32x4*>(A + a_base + (long long)row * lda + k0 + kc);
    }
    if (B_KN) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            int unit = tid + 256 * u;
            int nc = (unit & 31) * 8, kg = (unit >> 5) * 4;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                s.b[u * 4 + j] = *reinterpret_cast<const rv_u32x4*>(B + b_base + (long long)(k0 + kg + j) * ldb + nc);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int v = tid + 256 * i;
            int row = v >> 3, kc = (v & 7) * 8;
            s.b[i] = *reinterpret_cast<const rv_u32x4*>(B + b_base + (long long)row * ldb + k0 + kc);
        }
    }
}

// Writes half `h` (0 or 1) of the prefetched registers into an LDS stage.
template <bool B_KN>
__device__ __forceinline__ void rv_g2_store(const rv_g2_regs<B_KN>& s, unsigned short* As, unsigned short* Bs, int tid,
                                            int h) {
#pragma unroll
    for (int i = 4 * h; i < 4 * h + 4; ++i) {
        int v = tid + 256 * i;
        int row = v >> 3, kc = (v & 7) * 8;
        *reinterpret_cast<rv_u32x4*>(As + row * RV_G2_LDK + kc) = s.a[i];
    }
    if (B_KN) {
        const int u = h;
        int unit = tid + 256 * u;
        int nc = (unit & 31) * 8, kg = (unit >> 5) * 4;
        typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            int w = e >> 1;
            unsigned x0 = s.b[u * 4 + 0][w], x1 = s.b[u * 4 + 1][w], x2 = s.b[u * 4 + 2][w], x3 = s.b[u * 4 + 3][w];
            u32x2 pk;
            if (e & 1) {
                pk[0] = (x0 >> 16) | (x1 & 0xffff0000u);
                pk[1] = (x2 >> 16) | (x3 & 0xffff0000u);
            } else {
                pk[0] = (x0 & 0xffffu) | (x1 << 16);
                pk[1] = (x2 & 0xffffu) | (x3 << 16);
            }
            *reinterpret_cast<u32x2*>(Bs + (nc + e) * RV_G2_LDK + kg) = pk;
        }
    } else {
#pragma unroll
        for (int i = 4 * h; i < 4 * h + 4; ++i) {
            int v = tid + 256 * i;
            int row = v >> 3, kc = (v & 7) * 8;
            *reinterpret_cast<rv_u32x4*>(Bs + row * RV_G2_LDK + kc) = s.b[i];
        }
    }
}

template <class Acc>
__device__ __forceinline__ void rv_g2_mma(Acc& acc, const unsigned short* As, const unsigned short* Bs, int wm, int wn,
                                          int lane, int kk) {
    rv_bf16x8 af[4], bf[4];
    const int kq = kk + (lane >> 5) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const rv_bf16x8*>(As + (wm * 128 + i * 32 + (lane & 31)) * RV_G2_LDK + kq);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const rv_bf16x8*>(Bs + (wn * 128 + j * 32 + (lane & 31)) * RV_G2_LDK + kq);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
}

template <bool B_KN, int MODE, class Epi>
__device__ __forceinline__ void rv_gemm256_bf16(const unsigned short* __restrict__ A,
                                                const unsigned short* __restrict__ B, long long a_off, long long lda,
                                                long long b_off, long long ldb, int M, int N, int K, const Epi& epi,
                                                float* __restrict__ partials) {
    __shared__ __attribute__((aligned(16))) unsigned short lds_a[2][RV_G2_BM * RV_G2_LDK];
    __shared__ __attribute__((aligned(16))) unsigned short lds_b[2][RV_G2_BN * RV_G2_LDK];
    __shared__ float lds_red[4];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tiles_m = M / RV_G2_BM, tiles_n = N / RV_G2_BN;
    const int ntiles = tiles_m * tiles_n;
    int tm, tn;
    {
        int bid = blockIdx.x;
        if ((ntiles & 7) == 0 && (tiles_m & 3) == 0) {
            const int sb = (bid & 7) * (ntiles >> 3) + (bid >> 3);  // XCD-contiguous
            const int group = sb / (4 * tiles_n), within = sb % (4 * tiles_n);
            tm = group * 4 + (within & 3);
            tn = within >> 2;
        } else {
            tm = bid / tiles_n;
            tn = bid % tiles_n;
        }
    }
    const int m0 = tm * RV_G2_BM, n0 = tn * RV_G2_BN;
    const long long a_base = a_off + (long long)m0 * lda;
    const long long b_base = B_KN ? b_off + n0 : b_off + (long long)n0 * ldb;

    rv_f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    rv_g2_regs<B_KN> st;
    rv_g2_load<B_KN>(st, A, B, a_base, lda, b_base, ldb, 0, tid);
    rv_g2_store<B_KN>(st, lds_a[0], lds_b[0], tid, 0);
    rv_g2_store<B_KN>(st, lds_a[0], lds_b[0], tid, 1);
    __syncthreads();
    const int KT = K / RV_G2_BK;
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < KT;
        if (more) rv_g2_load<B_KN>(st, A, B, a_base, lda, b_base, ldb, (kt + 1) * RV_G2_BK, tid);
        rv_g2_mma(acc, lds_a[cur], lds_b[cur], wm, wn, lane, 0);
        rv_g2_mma(acc, lds_a[cur], lds_b[cur], wm, wn, lane, 16);
        if (more) rv_g2_store<B_KN>(st, lds_a[cur ^ 1], lds_b[cur ^ 1], tid, 0);
        rv_g2_mma(acc, lds_a[cur], lds_b[cur], wm, wn, lane, 32);
        rv_g2_mma(acc, lds_a[cur], lds_b[cur], wm, wn, lane, 48);
        if (more) rv_g2_store<B_KN>(st, lds_a[cur ^ 1], lds_b[cur ^ 1], tid, 1);
        __syncthreads();
    }

    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 128 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                const int n = n0 + wn * 128 + j * 32 + (lane & 31);
                const float v = epi(acc[i][j][r], m, n);
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
