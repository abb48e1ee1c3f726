// sgemm_kernels.hpp -- gfx950 (MI355X) FP32 SGEMM kernels.
//
// C = alpha * A * B + beta * C, row-major A (M x K), B (K x N), C (M x N),
// element (r, c) at r*ld + c ("如何高效实现矩阵乘？CUDA初学者的角度入门",
// section "樸素 GEMM 與前置知識").  Two inner products share one staging
// scheme:
//
//   * sgemm_valu: a register outer product on the vector ALU, each lane
//     accumulating a TM x TN micro-tile with FP32 FMA ("如何高效实现矩阵乘",
//     section "Thread 級優化", the outer-product form with one register of A
//     and a row of B registers per k).
//   * sgemm_mfma: v_mfma_f32_32x32x2_f32, each wave accumulating a WM x WN
//     wave tile in 32 x 32 blocks (16 accumulators per lane per block).
//
// Staging (both kernels).  The block tile walks K in steps of BK.  Per step:
//   1. global -> VGPR: A's BM x BK block and B's BK x BN block.  B is read
//      with 128-bit loads along N when VEC == 4, else with 32-bit loads.  A is
//      read as 4 rows x 1 column per thread: consecutive lanes walk K, so
//      every load instruction covers whole row segments of A.
//   2. VGPR -> LDS: A is stored TRANSPOSED (k-major, As[k][m]) with its rows
//      padded by PADA floats, one 128-bit store per 4 rows; B is stored as it
//      is (Bs[k][n], padded by PADB).  This is the layout of "SGEMM CUDA kernel
//      (Second Half)", Part 8 "Transposed As": A read as 4 x 1, written as a
//      1 x 4 vector into a transposed tile whose rows are shifted by 4 extra
//      columns so that the vector stores do not collide in LDS banks.  With
//      SWZ the rows are not padded and the columns are XOR-permuted instead
//      (see swz_col below); the large-shape tile uses that form.
//   3. Two LDS stages: the global loads of step t+1 are issued before the
//      LDS reads and arithmetic of step t, and written to the other stage
//      afterwards; one workgroup barrier per step ("如何高效实现矩阵乘", section
//      "Double Buffer").
//
// Partial tiles ("3.3 Shared memory ו tiling תרגול", exercise 1: pad partial
// tiles with zeros).  With BUF (the normal case) every global access is a raw
// buffer access whose descriptor ends at the matrix's last element: reads
// past it return 0.0 and writes past it are dropped by the hardware, with no
// branch in the kernel.  What the descriptor cannot cut off is handled so:
//   * A columns k >= K inside the matrix get an out-of-range offset in the
//     last K tile, so they read 0.0 (they meet B rows k >= K, which also read
//     0.0, and 0 * 0 keeps NaN and Inf out);
//   * B columns n >= N inside the matrix are read as they are: they only feed
//     C columns >= N, which are never stored;
//   * C columns n >= N inside the matrix get an out-of-range offset.
// Without BUF (leading dimensions too large for 31-bit offsets inside one
// tile) every element is checked explicitly and loads 0.0 outside.
//
// Workgroup -> tile order: consecutive workgroup ids walk one row of C tiles
// (the M tile index is the slow one), "如何高效实现矩阵乘", section "Wave & L2
// cache Hit Rate".
//
// Nothing here includes or calls the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sgk {

#ifndef VALU_K_UNROLL
#define VALU_K_UNROLL 8
#endif

struct Args {
    int M, N, K;       // K == 0 here also when alpha == 0 (A and B not read)
    float alpha, beta;
    const float *A;
    const float *B;
    float *C;
    int64_t lda, ldb, ldc;
    // split-K only: number of K ranges, partial tiles [tile][split][BM*BN],
    // and the launch's phase (0: write partials, 1: sum them and store C;
    // stream-K: 2: whole tiles and workers' partial tiles, 3: sum them)
    int splits;
    float *partial;
    int phase;
    // stream-K only: tiles done whole (the first sk_whole in tile order) and
    // the workers that share the K tiles of the rest
    int sk_whole, sk_workers;
    // log2 of the device's XCD count: consecutive workgroup ids go to the
    // XCDs in turn
    int xcd_shift;
};

template <int W> struct vec_t;
template <> struct vec_t<1> { typedef float type; };
template <> struct vec_t<2> { typedef float2 type; };
template <> struct vec_t<4> { typedef float4 type; };

__device__ __forceinline__ float vget(float v, int) { return v; }
__device__ __forceinline__ float vget(const float2 &v, int i) { return i == 0 ? v.x : v.y; }
__device__ __forceinline__ float vget(const float4 &v, int i) {
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

typedef float floatx16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// Phase stamps, for a measurement build only (compiled with SGEMM_PHASES; in
// the library itself every method is empty and no code is generated).  Lane
// 0 of each workgroup's first wave records, per workgroup: the shader clock
// (s_memtime) at entry, after the first K tile has landed, after the K loop
// and after the epilogue's stores have completed; the sums over the K tiles
// of the tile body (MFMAs and the next tile's loads) and of the wait and
// barrier that end it; and the 100 MHz real-time clock at entry and at the
// end.  sgemm_phase_read copies the log out.
// ---------------------------------------------------------------------------
#ifdef SGEMM_PHASES
constexpr int kPhaseSlots = 8;
constexpr int kPhaseWorkgroups = 65536;
__device__ unsigned long long sgemm_phase_log[kPhaseWorkgroups * kPhaseSlots];

struct PhaseLog {
    unsigned long long t0 = 0, t1 = 0, body = 0, wait = 0;
    static __device__ __forceinline__ bool lead() { return threadIdx.x == 0 && blockIdx.x < kPhaseWorkgroups; }
    static __device__ __forceinline__ void put(int slot, unsigned long long v) {
        if (lead()) sgemm_phase_log[blockIdx.x * kPhaseSlots + slot] = v;
    }
    __device__ __forceinline__ void entry() {
        put(0, __builtin_amdgcn_s_memtime());
        put(6, __builtin_amdgcn_s_memrealtime());
    }
    __device__ __forceinline__ void landed() { put(1, __builtin_amdgcn_s_memtime()); }
    __device__ __forceinline__ void tile_begin() { t0 = __builtin_amdgcn_s_memtime(); }
    __device__ __forceinline__ void tile_mid() {
        t1 = __builtin_amdgcn_s_memtime();
        body += t1 - t0;
    }
    __device__ __forceinline__ void tile_end() { wait += __builtin_amdgcn_s_memtime() - t1; }
    __device__ __forceinline__ void looped() {
        put(2, __builtin_amdgcn_s_memtime());
        put(4, body);
        put(5, wait);
    }
    __device__ __forceinline__ void stored() {
        __builtin_amdgcn_s_waitcnt(0);  // the epilogue's stores have completed
        put(3, __builtin_amdgcn_s_memtime());
        put(7, __builtin_amdgcn_s_memrealtime());
    }
};
#else
struct PhaseLog {
    __device__ __forceinline__ void entry() {}
    __device__ __forceinline__ void landed() {}
    __device__ __forceinline__ void tile_begin() {}
    __device__ __forceinline__ void tile_mid() {}
    __device__ __forceinline__ void tile_end() {}
    __device__ __forceinline__ void looped() {}
    __device__ __forceinline__ void stored() {}
};
#endif

// ---------------------------------------------------------------------------
// Raw buffer accesses.  A descriptor covers [base, base + bytes); an access at
// a byte offset >= bytes reads 0 / writes nothing.  kOutOfRange is above every
// extent used here (extents are clamped below 2^31).
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const int n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, kRsrcWord3);
}

// The LLVM raw buffer intrinsics, bound by name with explicit vector types
// (the clang b64/b128 builtins of this toolchain lower to 32-bit loads).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ float raw_load_f32(rsrc_t, uint32_t, uint32_t, int) __asm("llvm.amdgcn.raw.ptr.buffer.load.f32");
__device__ f32x2 raw_load_v2f32(rsrc_t, uint32_t, uint32_t, int) __asm("llvm.amdgcn.raw.ptr.buffer.load.v2f32");
__device__ f32x4 raw_load_v4f32(rsrc_t, uint32_t, uint32_t, int) __asm("llvm.amdgcn.raw.ptr.buffer.load.v4f32");
__device__ void raw_store_f32(float, rsrc_t, uint32_t, uint32_t, int) __asm("llvm.amdgcn.raw.ptr.buffer.store.f32");
__device__ void raw_store_v2f32(f32x2, rsrc_t, uint32_t, uint32_t, int) __asm("llvm.amdgcn.raw.ptr.buffer.store.v2f32");
__device__ void raw_store_v4f32(f32x4, rsrc_t, uint32_t, uint32_t, int) __asm("llvm.amdgcn.raw.ptr.buffer.store.v4f32");

template <int W> struct buf;
template <> struct buf<1> {
    static __device__ __forceinline__ float load(rsrc_t r, uint32_t off, int aux = 0) {
        return raw_load_f32(r, off, 0, aux);
    }
    static __device__ __forceinline__ void store(float v, rsrc_t r, uint32_t off, int aux = 0) {
        raw_store_f32(v, r, off, 0, aux);
    }
};
template <> struct buf<2> {
    static __device__ __forceinline__ float2 load(rsrc_t r, uint32_t off, int aux = 0) {
        const f32x2 v = raw_load_v2f32(r, off, 0, aux);
        return make_float2(v.x, v.y);
    }
    static __device__ __forceinline__ void store(float2 v, rsrc_t r, uint32_t off, int aux = 0) {
        f32x2 u;
        u.x = v.x;
        u.y = v.y;
        raw_store_v2f32(u, r, off, 0, aux);
    }
};
template <> struct buf<4> {
    static __device__ __forceinline__ float4 load(rsrc_t r, uint32_t off, int aux = 0) {
        const f32x4 v = raw_load_v4f32(r, off, 0, aux);
        return make_float4(v.x, v.y, v.z, v.w);
    }
    static __device__ __forceinline__ void store(float4 v, rsrc_t r, uint32_t off, int aux = 0) {
        f32x4 u;
        u.x = v.x;
        u.y = v.y;
        u.z = v.z;
        u.w = v.w;
        raw_store_v4f32(u, r, off, 0, aux);
    }
};

// ---------------------------------------------------------------------------
// A tile: BM x BK block of A -> As[BK][BM + PADA] (transposed).
// Thread tid covers column tid % BK of rows r0 + {0..3} + p * ROWS_PER_PASS,
// r0 = 4 * (tid / BK), and writes one 128-bit LDS vector per 4 rows.
// ---------------------------------------------------------------------------
// The transposed store collides in LDS banks unless something breaks the
// power-of-two row stride.  "如何高效实现矩阵乘？CUDA初学者的角度入门", section
// "Shared Memory" / "128-bit conflict-free store", names two cures: pad the
// leading dimension by 4 (PADA above), or leave the tile unpadded and move
// the colliding data elsewhere by an index transform.  SWZ is a transform of
// the second kind, fitted to this store: the lanes that collide are the BK
// lanes writing the same 4-row chunk m of different rows k, so the 16-byte
// chunk index of row k is XORed with (k mod 16).  Sixteen consecutive k then
// hit sixteen different chunks (all 64 banks), no LDS is spent on padding,
// and each row stays a permutation of its own aligned 64-float groups, so an
// MFMA fragment read (one k, MI <= 4 consecutive m) stays one vector read.
__device__ __forceinline__ int swz_col(int k, int col) {
    return ((((col >> 2) ^ (k & 15))) << 2) | (col & 3);
}

template <int BM, int BK, int NT, int PADA, int STAGES, bool SWZ = false>
struct ATileGeom {
    static_assert(BM % 4 == 0, "BM must be a multiple of 4");
    static_assert(!SWZ || (BM % 64 == 0 && PADA == 0), "the swizzle permutes 64-float row blocks");
    static_assert(NT % BK == 0, "BK must divide the thread count");
    static constexpr int ROWS_PER_PASS = 4 * (NT / BK);
    static_assert(BM % ROWS_PER_PASS == 0, "A tile must divide evenly over the threads");
    static constexpr int PER = BM / ROWS_PER_PASS;
    static constexpr int SA = BM + PADA;

    float4 reg[STAGES][PER];  // register stages: K tiles in flight

    template <int S>
    __device__ __forceinline__ void store(float *As, int tid) const {
#pragma unroll
        for (int p = 0; p < PER; ++p) store_piece<S>(As, tid, p);
    }

    // one 128-bit LDS store: rows 4 (tid / BK) + p ROWS_PER_PASS + {0..3}
    template <int S>
    __device__ __forceinline__ void store_piece(float *As, int tid, int p) const {
        const int k = tid % BK;
        const int m = 4 * (tid / BK) + p * ROWS_PER_PASS;
        *reinterpret_cast<float4 *>(As + k * SA + (SWZ ? swz_col(k, m) : m)) = reg[S][p];
    }
};

template <int BM, int BK, int NT, int PADA, int STAGES, bool SWZ>
struct ATileBuf : ATileGeom<BM, BK, NT, PADA, STAGES, SWZ> {
    typedef ATileGeom<BM, BK, NT, PADA, STAGES, SWZ> G;
    rsrc_t rsrc;       // rows bm.. of A, up to A's last element
    uint32_t off[4];   // ((r0 + c) * lda + col) * 4
    uint32_t pass;     // ROWS_PER_PASS * lda * 4
    int col;

    __device__ __forceinline__ void init(const Args &a, int bm, int tid) {
        col = tid % BK;
        const int r0 = 4 * (tid / BK);
#pragma unroll
        for (int c = 0; c < 4; ++c) off[c] = (uint32_t)(((int64_t)(r0 + c) * a.lda + col) * 4);
        pass = (uint32_t)(G::ROWS_PER_PASS * a.lda * 4);
        rsrc = make_rsrc(a.A + (int64_t)bm * a.lda, ((int64_t)(a.M - bm - 1) * a.lda + a.K) * 4);
    }

    template <int S>
    __device__ __forceinline__ void load(const Args &a, int bm, int k0) {
#pragma unroll
        for (int p = 0; p < G::PER; ++p) load_piece<S>(a, bm, k0, p);
    }

    // the 4 rows of one 128-bit LDS store (rows >= M and columns >= K read 0.0)
    template <int S>
    __device__ __forceinline__ void load_piece(const Args &a, int, int k0, int p) {
        const bool kin = (k0 + col) < a.K;
        uint32_t o[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) o[c] = kin ? off[c] + 4u * (uint32_t)k0 + p * pass : kOutOfRange;
        G::reg[S][p].x = buf<1>::load(rsrc, o[0]);
        G::reg[S][p].y = buf<1>::load(rsrc, o[1]);
        G::reg[S][p].z = buf<1>::load(rsrc, o[2]);
        G::reg[S][p].w = buf<1>::load(rsrc, o[3]);
    }
};

template <int BM, int BK, int NT, int PADA, int STAGES, bool SWZ>
struct ATilePtr : ATileGeom<BM, BK, NT, PADA, STAGES, SWZ> {
    typedef ATileGeom<BM, BK, NT, PADA, STAGES, SWZ> G;
    int col, r0;

    __device__ __forceinline__ void init(const Args &, int, int tid) {
        col = tid % BK;
        r0 = 4 * (tid / BK);
    }

    template <int S>
    __device__ __forceinline__ void load(const Args &a, int bm, int k0) {
#pragma unroll
        for (int p = 0; p < G::PER; ++p) load_piece<S>(a, bm, k0, p);
    }

    // The lane's column and first row pass through an empty asm at each
    // load, so the compiler recomputes the 64-bit row addresses here instead
    // of hoisting one per row out of the K loop into registers.
    template <int S>
    __device__ __forceinline__ void load_piece(const Args &a, int bm, int k0, int p) {
        int c_ = col, r_ = r0;
        asm volatile("" : "+v"(c_), "+v"(r_));
        const bool kin = (k0 + c_) < a.K;
        const int row = bm + r_ + p * G::ROWS_PER_PASS;
        const float *q = a.A + (int64_t)row * a.lda + k0 + c_;
        const int rl = a.M - row;
        G::reg[S][p].x = (kin && rl > 0) ? q[0] : 0.0f;
        G::reg[S][p].y = (kin && rl > 1) ? q[a.lda] : 0.0f;
        G::reg[S][p].z = (kin && rl > 2) ? q[2 * a.lda] : 0.0f;
        G::reg[S][p].w = (kin && rl > 3) ? q[3 * a.lda] : 0.0f;
    }
};

// ---------------------------------------------------------------------------
// B tile: BK x BN block of B -> Bs[BK][BN + PADB] (as is), VEC floats per
// load.  Consecutive threads take consecutive VEC-wide pieces of a row; piece
// p of a thread sits at tile row k_first + dk(p), tile column n_first + dn(p).
// ---------------------------------------------------------------------------
template <int BN, int BK, int NT, int PADB, int VEC, int STAGES>
struct BTileGeom {
    static constexpr int PER_ROW = BN / VEC;
    static_assert(BN % VEC == 0, "BN must be a multiple of VEC");
    static_assert(NT % PER_ROW == 0 || PER_ROW % NT == 0, "B tile rows and threads must nest");
    static constexpr int ITEMS = BK * PER_ROW;
    static_assert(ITEMS % NT == 0, "B tile must divide evenly over the threads");
    static constexpr int PER = ITEMS / NT;
    static constexpr int SB = BN + PADB;
    typedef typename vec_t<VEC>::type V;

    V reg[STAGES][PER];  // register stages: K tiles in flight

    static __device__ __forceinline__ constexpr int dk(int p) {
        return NT % PER_ROW == 0 ? p * (NT / PER_ROW) : (p * NT) / PER_ROW;
    }
    static __device__ __forceinline__ constexpr int dn(int p) {
        return NT % PER_ROW == 0 ? 0 : ((p * NT) % PER_ROW) * VEC;
    }

    template <int S>
    __device__ __forceinline__ void store(float *Bs, int tid) const {
#pragma unroll
        for (int p = 0; p < PER; ++p) store_piece<S>(Bs, tid, p);
    }

    template <int S>
    __device__ __forceinline__ void store_piece(float *Bs, int tid, int p) const {
        float *dst = Bs + (tid / PER_ROW) * SB + (tid % PER_ROW) * VEC;
        *reinterpret_cast<V *>(dst + dk(p) * SB + dn(p)) = reg[S][p];
    }
};

template <int BN, int BK, int NT, int PADB, int VEC, int STAGES>
struct BTileBuf : BTileGeom<BN, BK, NT, PADB, VEC, STAGES> {
    typedef BTileGeom<BN, BK, NT, PADB, VEC, STAGES> G;
    uint32_t off;  // (k_first * ldb + n_first) * 4
    uint32_t ldb4;

    __device__ __forceinline__ void init(const Args &a, int, int tid) {
        const int k_first = tid / G::PER_ROW;
        const int n_first = (tid % G::PER_ROW) * VEC;
        off = (uint32_t)(((int64_t)k_first * a.ldb + n_first) * 4);
        ldb4 = (uint32_t)(a.ldb * 4);
    }

    template <int S>
    __device__ __forceinline__ void load(const Args &a, int bn, int k0) {
        // Rows k0.. of B from column bn, up to B's last element: rows >= K
        // read 0.0.  With VEC == 4, N and ldb are multiples of 4, so no
        // 128-bit piece straddles the end.
        const rsrc_t r = rows(a, bn, k0);
#pragma unroll
        for (int p = 0; p < G::PER; ++p)
            G::reg[S][p] = buf<VEC>::load(r, off + G::dk(p) * ldb4 + G::dn(p) * 4);
    }

    __device__ __forceinline__ rsrc_t rows(const Args &a, int bn, int k0) const {
        return make_rsrc(a.B + (int64_t)k0 * a.ldb + bn, ((int64_t)(a.K - k0 - 1) * a.ldb + (a.N - bn)) * 4);
    }

    template <int S>
    __device__ __forceinline__ void load_piece(const Args &a, int bn, int k0, int p) {
        G::reg[S][p] = buf<VEC>::load(rows(a, bn, k0), off + G::dk(p) * ldb4 + G::dn(p) * 4);
    }
};

template <int BN, int BK, int NT, int PADB, int VEC, int STAGES>
struct BTilePtr : BTileGeom<BN, BK, NT, PADB, VEC, STAGES> {
    typedef BTileGeom<BN, BK, NT, PADB, VEC, STAGES> G;
    int k_first, n_first;

    __device__ __forceinline__ void init(const Args &, int, int tid) {
        k_first = tid / G::PER_ROW;
        n_first = (tid % G::PER_ROW) * VEC;
    }

    template <int S>
    __device__ __forceinline__ void load(const Args &a, int bn, int k0) {
#pragma unroll
        for (int p = 0; p < G::PER; ++p) load_piece<S>(a, bn, k0, p);
    }

    // As in ATilePtr: the lane's coordinates are opaque at each load.
    template <int S>
    __device__ __forceinline__ void load_piece(const Args &a, int bn, int k0, int p) {
        int nf = n_first, kf = k_first;
        asm volatile("" : "+v"(nf), "+v"(kf));
        const int n = bn + nf + G::dn(p);
        const int k = k0 + kf + G::dk(p);
        // VEC == 4 only when N % 4 == 0: a piece is all in or all out
        if (n < a.N && k < a.K)
            G::reg[S][p] = *reinterpret_cast<const typename G::V *>(a.B + (int64_t)k * a.ldb + n);
        else
            G::reg[S][p] = typename G::V{};
    }
};

// ---------------------------------------------------------------------------
// Epilogue: C = alpha*acc + beta*C (C read only when beta != 0).  VEC == 4
// means N, ldc and C are 16-byte friendly, so a W-wide group at a multiple of
// W is wholly inside or wholly outside the matrix and moves as one vector.
// ---------------------------------------------------------------------------
// C accesses of the epilogue, W consecutive columns of one row at tile
// coordinates (r, c).  load() reads the old values (only called when
// beta != 0); store() writes the new ones; both skip what lies outside C.
//
// Buffered: rc covers rows bm.. of C from column bn up to C's last element.
// C is read and written once per launch, so its accesses carry the
// non-temporal cache policy (the auxiliary operand of the buffer intrinsics:
// bit 1, NT on gfx950), which leaves L2 to the A and B tiles that are reused:
// 1.3-2.4% faster at 16384^2 x 128 with beta = 1, no change at 8192^3.
constexpr int kCPolStream = 2;

template <int W, int VEC, int CPOL = kCPolStream>
struct CStoreBuf {
    rsrc_t rc;
    int ncols;  // N - bn

    __device__ __forceinline__ void init(const Args &a, int bm, int bn) {
        rc = make_rsrc(a.C + (int64_t)bm * a.ldc + bn, ((int64_t)(a.M - bm - 1) * a.ldc + (a.N - bn)) * 4);
        ncols = a.N - bn;
    }

    __device__ __forceinline__ uint32_t offset(const Args &a, int r, int c) const {
        return (uint32_t)(((int64_t)r * a.ldc + c) * 4);
    }

    __device__ __forceinline__ void load(const Args &a, int r, int c, float (&old)[W]) const {
        load_if(true, a, r, c, old);
    }

    // With en == false every access is out of range: it reads 0.0 and touches no memory.
    __device__ __forceinline__ void load_if(bool en, const Args &a, int r, int c, float (&old)[W]) const {
        const uint32_t off = offset(a, r, c);
        if (VEC == 4 || W == 1) {
            const typename vec_t<W>::type v = buf<W>::load(rc, en && c < ncols ? off : kOutOfRange, CPOL);
#pragma unroll
            for (int i = 0; i < W; ++i) old[i] = vget(v, i);
        } else {
#pragma unroll
            for (int i = 0; i < W; ++i)
                old[i] = buf<1>::load(rc, en && c + i < ncols ? off + 4u * i : kOutOfRange, CPOL);
        }
    }

    __device__ __forceinline__ void store(const Args &a, int r, int c, const float (&out)[W]) const {
        const uint32_t off = offset(a, r, c);
        if (VEC == 4 || W == 1) {
            typename vec_t<W>::type v;
            float *o = reinterpret_cast<float *>(&v);
#pragma unroll
            for (int i = 0; i < W; ++i) o[i] = out[i];
            buf<W>::store(v, rc, c < ncols ? off : kOutOfRange, CPOL);
        } else {
#pragma unroll
            for (int i = 0; i < W; ++i) buf<1>::store(out[i], rc, c + i < ncols ? off + 4u * i : kOutOfRange, CPOL);
        }
    }
};

template <int W, int VEC>
struct CStorePtr {
    int bm, bn;

    __device__ __forceinline__ void init(const Args &, int bm_, int bn_) {
        bm = bm_;
        bn = bn_;
    }

    __device__ __forceinline__ void load(const Args &a, int r, int c, float (&old)[W]) const {
        load_if(true, a, r, c, old);
    }

    __device__ __forceinline__ void load_if(bool en, const Args &a, int r, int c, float (&old)[W]) const {
        const int row = bm + r, col = bn + c;
        const float *p = a.C + (int64_t)row * a.ldc + col;
#pragma unroll
        for (int i = 0; i < W; ++i) old[i] = (en && row < a.M && col + i < a.N) ? p[i] : 0.0f;
    }

    __device__ __forceinline__ void store(const Args &a, int r, int c, const float (&out)[W]) const {
        const int row = bm + r, col = bn + c;
        if (row >= a.M) return;
        float *p = a.C + (int64_t)row * a.ldc + col;
        if (VEC == 4 && W > 1) {
            if (col >= a.N) return;
            typename vec_t<W>::type v;
            float *o = reinterpret_cast<float *>(&v);
#pragma unroll
            for (int i = 0; i < W; ++i) o[i] = out[i];
            *reinterpret_cast<typename vec_t<W>::type *>(p) = v;
        } else {
#pragma unroll
            for (int i = 0; i < W; ++i)
                if (col + i < a.N) p[i] = out[i];
        }
    }
};

// The epilogue proper: NV vectors of W columns per lane, vector v at tile
// coordinates pos(v) with values val(v).  beta is uniform, so the test is
// taken once; with beta != 0 the old values of G vectors are requested
// together before any of them is combined and stored, so the loads' latency
// is paid once per group instead of once per vector (a group holds GV old
// values: GV extra VGPRs at most).
template <int NV, int W, class TC, class Pos, class Val, int GV = 32>
__device__ __forceinline__ void epilogue(const Args &a, const TC &st, Pos pos, Val val) {
    if (a.beta != 0.0f) {
        constexpr int G = NV < GV / W ? NV : (GV / W > 0 ? GV / W : 1);
        static_assert(NV % G == 0, "epilogue groups");
#pragma unroll
        for (int b = 0; b < NV; b += G) {
            float old[G][W];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                int r, c;
                pos(b + g, r, c);
                st.load(a, r, c, old[g]);
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                int r, c;
                pos(b + g, r, c);
                float v[W], out[W];
                val(b + g, v);
#pragma unroll
                for (int i = 0; i < W; ++i) out[i] = fmaf(a.alpha, v[i], a.beta * old[g][i]);
                st.store(a, r, c, out);
            }
        }
    } else {
#pragma unroll
        for (int b = 0; b < NV; ++b) {
            int r, c;
            pos(b, r, c);
            float v[W], out[W];
            val(b, v);
#pragma unroll
            for (int i = 0; i < W; ++i) out[i] = a.alpha * v[i];
            st.store(a, r, c, out);
        }
    }
}

// The same with the old values of vectors 0 .. NP - 1 already in pre (read
// before the K loop ended); NP is a whole number of groups.
template <int NV, int W, class TC, class Pos, class Val, int GV, int NP>
__device__ __forceinline__ void epilogue_pre(const Args &a, const TC &st, Pos pos, Val val,
                                             const float (&pre)[NP][W]) {
    constexpr int G = NV < GV / W ? NV : (GV / W > 0 ? GV / W : 1);
    static_assert(NV % G == 0 && NP % G == 0 && NP <= NV, "epilogue groups");
    if (a.beta != 0.0f) {
#pragma unroll
        for (int b = 0; b < NV; b += G) {
            float old[G][W];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (b + g < NP) {
#pragma unroll
                    for (int i = 0; i < W; ++i) old[g][i] = pre[b + g < NP ? b + g : 0][i];
                } else {
                    int r, c;
                    pos(b + g, r, c);
                    st.load(a, r, c, old[g]);
                }
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                int r, c;
                pos(b + g, r, c);
                float v[W], out[W];
                val(b + g, v);
#pragma unroll
                for (int i = 0; i < W; ++i) out[i] = fmaf(a.alpha, v[i], a.beta * old[g][i]);
                st.store(a, r, c, out);
            }
        }
    } else {
        epilogue<NV, W, TC, Pos, Val, GV>(a, st, pos, val);
    }
}

template <bool BUF, int BM, int BN, int BK, int NT, int PADA, int PADB, int VEC, int W, int STAGES,
          bool SWZ = false>
struct Staging {
    typedef typename std::conditional<BUF, ATileBuf<BM, BK, NT, PADA, STAGES, SWZ>,
                                      ATilePtr<BM, BK, NT, PADA, STAGES, SWZ>>::type TA;
    typedef typename std::conditional<BUF, BTileBuf<BN, BK, NT, PADB, VEC, STAGES>,
                                      BTilePtr<BN, BK, NT, PADB, VEC, STAGES>>::type TB;
    typedef typename std::conditional<BUF, CStoreBuf<W, VEC>, CStorePtr<W, VEC>>::type TC;
};

// ---------------------------------------------------------------------------
// VALU kernel.  Block tile BM x BN, NT = (BM / (8*TM)) * (BN / (8*TN)) * 64.
// A wave owns an (8*TM) x (8*TN) tile; lane (ly, lx) = (lane / 8, lane % 8)
// owns rows  wm + 4*ly + {0..3} + 32*s  (s < TM/4)  and
//      cols  wn + 4*lx + {0..3} + 32*s  (s < TN/4),
// so every LDS read is one 128-bit load that 8 lanes share (broadcast).
// ---------------------------------------------------------------------------
template <int BM, int BN, int BK, int TM, int TN, int PADA, int PADB, int VEC, int WPE, bool BUF>
__global__ void __launch_bounds__((BM / (8 * TM)) * (BN / (8 * TN)) * 64)
__attribute__((amdgpu_waves_per_eu(WPE))) sgemm_valu(Args a) {
    constexpr int WM = 8 * TM, WN = 8 * TN;
    constexpr int WAVES_N = BN / WN;
    constexpr int NT = (BM / WM) * WAVES_N * 64;
    static_assert(TM % 4 == 0 && TN % 4 == 0, "micro-tile sides must be multiples of 4");
    constexpr int SA = BM + PADA, SB = BN + PADB;
    constexpr int STAGE = BK * (SA + SB);
    typedef Staging<BUF, BM, BN, BK, NT, PADA, PADB, VEC, 4, 1> S;
    __shared__ __attribute__((aligned(16))) float smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int nbn = (a.N + BN - 1) / BN;
    const int bm = (int)(blockIdx.x / nbn) * BM;
    const int bn = (int)(blockIdx.x % nbn) * BN;
    const int wm = (wave / WAVES_N) * WM, wn = (wave % WAVES_N) * WN;
    const int ly = lane >> 3, lx = lane & 7;

    typename S::TA ta;
    typename S::TB tb;
    ta.init(a, bm, tid);
    tb.init(a, bn, tid);

    float acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = 0.0f;

    const int KT = (a.K + BK - 1) / BK;
    if (KT > 0) {
        ta.template load<0>(a, bm, 0);
        tb.template load<0>(a, bn, 0);
        ta.template store<0>(smem, tid);
        tb.template store<0>(smem + BK * SA, tid);
    }
    __syncthreads();

    for (int t = 0; t < KT; ++t) {
        const float *As = smem + (t & 1) * STAGE;
        const float *Bs = As + BK * SA;
        if (t + 1 < KT) {
            ta.template load<0>(a, bm, (t + 1) * BK);
            tb.template load<0>(a, bn, (t + 1) * BK);
        }
        const float *ap = As + wm + 4 * ly;
        const float *bp = Bs + wn + 4 * lx;
        // Partial unrolling bounds how many k-steps of fragments the compiler
        // hoists ahead of their FMAs (a full unroll costs 16 VGPRs per step).
#pragma unroll VALU_K_UNROLL
        for (int k = 0; k < BK; ++k) {
            float ra[TM], rb[TN];
#pragma unroll
            for (int s = 0; s < TM / 4; ++s)
                *reinterpret_cast<float4 *>(&ra[4 * s]) =
                    *reinterpret_cast<const float4 *>(ap + k * SA + 32 * s);
#pragma unroll
            for (int s = 0; s < TN / 4; ++s)
                *reinterpret_cast<float4 *>(&rb[4 * s]) =
                    *reinterpret_cast<const float4 *>(bp + k * SB + 32 * s);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = fmaf(ra[i], rb[j], acc[i][j]);
        }
        if (t + 1 < KT) {
            float *An = smem + ((t + 1) & 1) * STAGE;
            ta.template store<0>(An, tid);
            tb.template store<0>(An + BK * SA, tid);
        }
        __syncthreads();
    }

    // 8 lanes with the same ly cover 32 consecutive columns (128 bytes) of a row;
    // vector v is micro-tile row v / (TN/4), column group v % (TN/4)
    typename S::TC st;
    st.init(a, bm, bn);
    constexpr int CG = TN / 4;
    auto pos = [&](int v, int &r, int &c) {
        const int i = v / CG, g = v % CG;
        r = wm + 4 * ly + (i & 3) + 32 * (i >> 2);
        c = wn + 4 * lx + 32 * g;
    };
    auto val = [&](int v, float (&x)[4]) {
        const int i = v / CG, g = v % CG;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc[i][4 * g + e];
    };
    // 32-bit accesses take 4 loads per vector: fewer old values in flight
    // (beta != 0) keep the 8 x 8 tile within its 128 registers
    epilogue<TM * CG, 4, typename S::TC, decltype(pos), decltype(val), VEC == 4 ? 32 : 16>(a, st, pos, val);
}

// ---------------------------------------------------------------------------
// MFMA kernel.  Block tile BM x BN, waves of WM x WN, NT = (BM/WM)*(BN/WN)*64,
// at least WPE waves per SIMD (1 lets a wave use all 512 registers).
// v_mfma_f32_32x32x2_f32 takes from lane l the A element (row l%32, k l/32)
// and the B element (k l/32, col l%32), and leaves the 32 x 32 result with
// lane l holding column l%32, rows 8*(r/4) + 4*(l/32) + r%4 in accumulator
// register r (r < 16).
//
// A wave tile is MI x NI such blocks (MI = WM/32, NI = WN/32).  Block (mi, ni)
// row i is tile row MI*i + mi, column j is tile column NI*j + ni, so one
// MI-wide LDS load at As[k][wm + MI*i] gives lane i its A element for every
// mi, and one NI-wide load gives its B elements for every ni.  In the
// epilogue the NI accumulators of one register index are NI consecutive
// columns, so each lane stores NI-wide vectors and 32 lanes cover 32*NI
// consecutive columns of a row.
//
// The fragments of k-step j+1 are read from LDS while the MFMAs of step j
// issue, so the LDS latency hides behind matrix work.
// ---------------------------------------------------------------------------
// Workgroup -> C tile.  ORDER 0: row-major over tiles, the M index slow
// ("如何高效实现矩阵乘", section "Wave & L2 cache Hit Rate").  ORDER 1: the
// same tiles, assigned so that each XCD works on a compact patch.  MI355X
// hands consecutive workgroup ids to its X XCDs in turn (id % X), and each
// XCD has its own L2; the id is first renumbered so that every XCD receives
// a contiguous run of the tile sequence, and the sequence then walks groups
// of GROUP_M tile rows column by column, so the workgroups an XCD runs at
// once share GROUP_M row blocks of A and a few column blocks of B.
// ORDER 2: row-major as seen from each XCD.  With the tile columns a multiple
// of X, row-major dealing already gives XCD x the columns x, x + X, ... in
// every row, and this order is the same mapping.  Otherwise the column an
// XCD receives shifts from row to row and the workgroups it runs at once
// need up to X times as many B column blocks; here XCD x keeps the columns
// x, x + X, ... below X floor(nbn / X) and walks them row by row, and the
// remaining nbn mod X columns, row-major, are dealt out last in one
// contiguous run per XCD.  X = 2^xs is the device's XCD count (8 on an
// MI355X, 4, 2 or 1 on its partitions: a power of two, so no division by
// it is needed; X = 1 makes every order row-major).  Every order is a
// bijection of [0, nbm nbn) onto the tiles.
template <int ORDER, int GROUP_M>
__host__ __device__ __forceinline__ void tile_of(int pid, int nbm, int nbn, int xs, int &tm, int &tn) {
    const int X = 1 << xs;
    if (ORDER == 0 || X == 1) {
        tm = pid / nbn;
        tn = pid % nbn;
        return;
    }
    const int c = nbn >> xs, rem = nbn & (X - 1);
    if (ORDER == 2 && (rem == 0 || c == 0)) {
        tm = pid / nbn;
        tn = pid % nbn;
        return;
    }
    const int total = nbm * nbn;
    const int q = total >> xs, r = total & (X - 1);
    const int x = pid & (X - 1), idx = pid >> xs;
    if (ORDER == 2) {
        const int common = nbm * c;  // tiles of XCD x in its own columns
        if (idx < common) {
            tm = idx / c;
            tn = x + X * (idx - tm * c);
            return;
        }
        // XCDs before x hold x q + min(x, r) ids, x * common of them in
        // their own columns; the rest index the remaining columns' tiles
        const int g = x * q + (x < r ? x : r) - x * common + (idx - common);
        tm = g / rem;
        tn = X * c + (g - tm * rem);
        return;
    }
    // XCD x received ids x, x + X, ...: q + (x < r) of them
    const int seq = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + idx;
    const int per_group = GROUP_M * nbn;
    const int group = seq / per_group;
    const int first_m = group * GROUP_M;
    const int rows = nbm - first_m < GROUP_M ? nbm - first_m : GROUP_M;
    const int in_group = seq - group * per_group;
    tm = first_m + in_group % rows;
    tn = in_group / rows;
}

// One K tile of MFMAs from one LDS stage.  The fragments of k-step j + FD
// are read while the MFMAs of step j issue, so the LDS latency hides behind
// FD steps of matrix work (FD > 1 for wave tiles with few MFMAs per step).
// With CH == 2 the odd k-steps accumulate into acc_odd: a wave with a single
// 32 x 32 block (MI = NI = 1) otherwise issues a chain of MFMAs that each wait
// for the previous one's result.  The caller adds acc_odd into acc once, after
// the K loop.
struct NoHook {
    __device__ __forceinline__ void operator()(int, int) const {}
};

// hook(j, u) runs after MFMA u of k-step j (u = i * NI + jj), fenced so that
// it stays there: other work (the next K tile's global loads and LDS stores)
// issued while the matrix pipe is busy instead of before or after the MFMAs.
template <int BK, int MI, int NI, int SA, int SB, int FD, bool SWZ, int CH = 1, class Hook = NoHook>
__device__ __forceinline__ void mfma_tile(const float *as, int a_col, int lh, const float *bp,
                                          floatx16 (&acc)[MI][NI], floatx16 (&acc_odd)[MI][NI],
                                          Hook hook = Hook()) {
    constexpr bool HOOKED = !std::is_same<Hook, NoHook>::value;
    typedef typename vec_t<MI>::type VA;
    typedef typename vec_t<NI>::type VB;
    constexpr int STEPS = BK / 2;
    constexpr int RING = FD + 1;
    // A fragment of k-step j: LDS row 2j + lh, column a_col (swizzled or not)
    auto a_at = [&](int j) -> const VA * {
        const int row = 2 * j + lh;
        return reinterpret_cast<const VA *>(as + row * SA + (SWZ ? swz_col(row, a_col) : a_col));
    };
    VA av[RING];
    VB bv[RING];
#pragma unroll
    for (int f = 0; f < FD && f < STEPS; ++f) {
        av[f] = *a_at(f);
        bv[f] = *reinterpret_cast<const VB *>(bp + 2 * f * SB);
    }
#pragma unroll
    for (int j = 0; j < STEPS; ++j) {
        if (j + FD < STEPS) {
            av[(j + FD) % RING] = *a_at(j + FD);
            bv[(j + FD) % RING] = *reinterpret_cast<const VB *>(bp + 2 * (j + FD) * SB);
        }
        // Keep the early reads above this step's MFMAs: without the fence the
        // scheduler sinks each read next to its first use and waits on it.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int jj = 0; jj < NI; ++jj) {
                if (CH == 2 && (j & 1))
                    acc_odd[i][jj] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                        vget(av[j % RING], i), vget(bv[j % RING], jj), acc_odd[i][jj], 0, 0, 0);
                else
                    acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                        vget(av[j % RING], i), vget(bv[j % RING], jj), acc[i][jj], 0, 0, 0);
                if (HOOKED) {
                    __builtin_amdgcn_sched_barrier(0);
                    hook(j, i * NI + jj);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
    }
}

template <int BK, int MI, int NI, int SA, int SB, int FD, bool SWZ>
__device__ __forceinline__ void mfma_tile(const float *as, int a_col, int lh, const float *bp,
                                          floatx16 (&acc)[MI][NI]) {
    mfma_tile<BK, MI, NI, SA, SB, FD, SWZ, 1>(as, a_col, lh, bp, acc, acc);
}

// Epilogue of a wave's MI x NI accumulator blocks: register r of block
// (mi, ni) on lane (li, lh) is tile row wm + MI*(8*(r/4) + 4*lh + r%4) + mi,
// tile column wn + NI*li + ni.
// GV bounds the old C values requested at once when beta != 0.
template <class S, int MI, int NI, int GV = 32>
__device__ __forceinline__ void epilogue_mfma(const Args &a, int bm, int bn, int wm, int wn, int li,
                                              int lh, const floatx16 (&acc)[MI][NI]) {
    typename S::TC st;
    st.init(a, bm, bn);
    // vector v is accumulator register v % 16 of block row v / 16
    auto pos = [&](int v, int &r, int &c) {
        const int i = v / 16, reg = v % 16;
        r = wm + MI * (8 * (reg >> 2) + 4 * lh + (reg & 3)) + i;
        c = wn + NI * li;
    };
    auto val = [&](int v, float (&x)[NI]) {
#pragma unroll
        for (int j = 0; j < NI; ++j) x[j] = acc[v / 16][j][v % 16];
    };
    epilogue<MI * 16, NI, typename S::TC, decltype(pos), decltype(val), GV>(a, st, pos, val);
}

// Epilogue through LDS ("SGEMM CUDA kernel (Second Half)", Part 9: each warp
// stages its results in a shared buffer and flushes whole rows with
// coalesced stores).  Each wave stages 16 of its tile rows at a time in its
// own LDS area (16 x (WN + 4) floats), then its 64 lanes read them back as
// 4-float vectors in row order and store them, so one store instruction
// covers 64 x 16 contiguous-in-row bytes (whole rows of the wave tile).  The
// direct epilogue already stores 32 x 4 x NI contiguous bytes per row; this
// variant exists to measure the difference on MI355X.
template <class TC4, int MI, int NI, int WN>
__device__ __forceinline__ void epilogue_mfma_staged(const Args &a, const TC4 &st4, float *lds_wave,
                                                     int wm, int wn, int li, int lh, int lane,
                                                     const floatx16 (&acc)[MI][NI]) {
    typedef typename vec_t<NI>::type VB;
    constexpr int SW = WN + 4;
    constexpr int ROW4 = WN / 4;             // 4-float vectors per staged row
    constexpr int F4 = 16 * ROW4 / 64;       // vectors per lane per 16-row chunk
    static_assert((16 * ROW4) % 64 == 0, "staged chunk must split over 64 lanes");
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            __syncthreads();  // the previous chunk's reads are done
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int reg = 8 * h + q;
                const int lr = 8 * (reg >> 2) + 4 * lh + (reg & 3) - 16 * h;  // 0..15
                VB v;
                float *pv = reinterpret_cast<float *>(&v);
#pragma unroll
                for (int j = 0; j < NI; ++j) pv[j] = acc[mi][j][reg];
                *reinterpret_cast<VB *>(lds_wave + lr * SW + NI * li) = v;
            }
            __syncthreads();
            float4 vals[F4];
#pragma unroll
            for (int k = 0; k < F4; ++k) {
                const int f = lane + 64 * k;
                vals[k] = *reinterpret_cast<const float4 *>(lds_wave + (f / ROW4) * SW + 4 * (f % ROW4));
            }
            epilogue<F4, 4>(
                a, st4,
                [&](int k, int &r, int &c) {
                    const int f = lane + 64 * k;
                    r = wm + MI * (16 * h + f / ROW4) + mi;
                    c = wn + 4 * (f % ROW4);
                },
                [&](int k, float (&x)[4]) {
                    x[0] = vals[k].x;
                    x[1] = vals[k].y;
                    x[2] = vals[k].z;
                    x[3] = vals[k].w;
                });
        }
    }
}

// Register-staged MFMA kernel: the global loads of K tile t+1 land in
// registers and are stored to the other LDS stage (one register stage).  FD
// is the LDS fragment prefetch distance in k-steps.  IL selects the
// interleaved schedule (the loads and stores threaded between the MFMAs);
// otherwise the loads are issued before a tile's MFMAs and stored after them.
// EPI 1 takes the LDS-staged epilogue.  ORDER is the workgroup -> tile order
// of tile_of.
template <int BM, int BN, int BK, int WM, int WN, int PADA, int PADB, int VEC, int WPE, bool BUF,
          int FD, int ORDER, int EPI, bool SWZ, bool IL>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
__attribute__((amdgpu_waves_per_eu(WPE))) sgemm_mfma(Args a) {
    constexpr int MI = WM / 32, NI = WN / 32;
    constexpr int WAVES_N = BN / WN;
    constexpr int NT = (BM / WM) * WAVES_N * 64;
    constexpr int SA = BM + PADA, SB = BN + PADB;
    constexpr int STAGE = BK * (SA + SB);
    static_assert(BK % 2 == 0, "BK must be even (K = 2 per instruction)");
    static_assert(MI == 1 || MI == 2 || MI == 4, "MI in {1, 2, 4}");
    static_assert(NI == 1 || NI == 2 || NI == 4, "NI in {1, 2, 4}");
    typedef Staging<BUF, BM, BN, BK, NT, PADA, PADB, VEC, NI, 1, SWZ> S;
    __shared__ __attribute__((aligned(16))) float smem[2 * STAGE];

    PhaseLog ph;
    ph.entry();
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int nbm = (a.M + BM - 1) / BM, nbn = (a.N + BN - 1) / BN;
    int tm, tn;
    tile_of<ORDER, 8>((int)blockIdx.x, nbm, nbn, a.xcd_shift, tm, tn);
    const int bm = tm * BM, bn = tn * BN;
    const int wm = (wave / WAVES_N) * WM, wn = (wave % WAVES_N) * WN;
    const int li = lane & 31, lh = lane >> 5;

    typename S::TA ta;
    typename S::TB tb;
    ta.init(a, bm, tid);
    tb.init(a, bn, tid);

    // a lone 32 x 32 block per wave gets two accumulation chains (even and
    // odd k-steps), added together once after the K loop
    constexpr int CH = MI * NI == 1 ? 2 : 1;
    floatx16 acc[MI][NI], acc_odd[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = acc_odd[i][j][r] = 0.0f;

    // per-lane fragment bases inside one LDS stage
    const int a_col = wm + MI * li;
    const int b_off = BK * SA + lh * SB + wn + NI * li;
    const int KT = (a.K + BK - 1) / BK;

    if constexpr (IL) {
        // Interleaved schedule: the loads of K tile t+1 are issued in pieces
        // after the MFMAs of the first k-steps of tile t, and stored to the
        // other LDS stage in pieces over the last k-steps, so the matrix pipe
        // is fed throughout.  The loads are not conditional: after the last
        // tile they read past K, 0.0, into a stage nobody reads.
        constexpr int STEPS = BK / 2;
        constexpr int PA = S::TA::PER, PB = S::TB::PER, NP = PA + PB;
        // the first quarter of the k-steps carries the loads, the second half
        // the stores, one piece after every few MFMAs (spreading the pieces
        // over a step's MFMAs, rather than issuing them in one burst, was
        // worth 1.6%; with them spread, other splits measure the same)
        constexpr int LSTEPS = STEPS / 4 > 0 ? STEPS / 4 : 1;
        constexpr int SSTEPS = STEPS / 2 > 0 ? STEPS / 2 : 1;
        constexpr int LPER = (NP + LSTEPS - 1) / LSTEPS, SPER = (NP + SSTEPS - 1) / SSTEPS;
        if (KT > 0) {
            ta.template load<0>(a, bm, 0);
            tb.template load<0>(a, bn, 0);
            ta.template store<0>(smem, tid);
            tb.template store<0>(smem + BK * SA, tid);
        }
        __syncthreads();
        ph.landed();
        for (int t = 0; t < KT; ++t) {
            ph.tile_begin();
            const float *st = smem + (t & 1) * STAGE;
            float *nx = smem + ((t + 1) & 1) * STAGE;
            const int kn = (t + 1) * BK;
            // piece q of a step goes after MFMA (q * MI * NI) / pieces per step:
            // spread evenly, several after one MFMA when there are more
            // pieces than MFMAs
            constexpr int NU = MI * NI;
            auto hook = [&](int j, int u) {
                if (j < LSTEPS) {
#pragma unroll
                    for (int q = 0; q < LPER; ++q) {
                        const int piece = j * LPER + q;
                        if ((q * NU) / LPER != u || piece >= NP) continue;
                        if (piece < PA) ta.template load_piece<0>(a, bm, kn, piece);
                        else tb.template load_piece<0>(a, bn, kn, piece - PA);
                    }
                }
                if (j >= STEPS - SSTEPS) {
#pragma unroll
                    for (int q = 0; q < SPER; ++q) {
                        const int piece = (j - (STEPS - SSTEPS)) * SPER + q;
                        if ((q * NU) / SPER != u || piece >= NP) continue;
                        if (piece < PA) ta.template store_piece<0>(nx, tid, piece);
                        else tb.template store_piece<0>(nx + BK * SA, tid, piece - PA);
                    }
                }
            };
            mfma_tile<BK, MI, NI, SA, SB, FD, SWZ, CH>(st, a_col, lh, st + b_off, acc, acc_odd, hook);
            ph.tile_mid();
            __syncthreads();
            ph.tile_end();
        }
    } else {
        if (KT > 0) {
            ta.template load<0>(a, bm, 0);
            tb.template load<0>(a, bn, 0);
            ta.template store<0>(smem, tid);
            tb.template store<0>(smem + BK * SA, tid);
        }
        __syncthreads();
        ph.landed();
        for (int t = 0; t < KT; ++t) {
            ph.tile_begin();
            const float *st = smem + (t & 1) * STAGE;
            if (t + 1 < KT) {
                ta.template load<0>(a, bm, (t + 1) * BK);
                tb.template load<0>(a, bn, (t + 1) * BK);
            }
            mfma_tile<BK, MI, NI, SA, SB, FD, SWZ, CH>(st, a_col, lh, st + b_off, acc, acc_odd);
            if (t + 1 < KT) {
                float *nx = smem + ((t + 1) & 1) * STAGE;
                ta.template store<0>(nx, tid);
                tb.template store<0>(nx + BK * SA, tid);
            }
            ph.tile_mid();
            __syncthreads();
            ph.tile_end();
        }
    }
    ph.looped();

    if (CH == 2) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j) acc[i][j] += acc_odd[i][j];
    }

    if (EPI == 0) {
        // the checked C accesses are branches, each load waited for in its
        // own branch: few old values in flight, or they spill
        epilogue_mfma<S, MI, NI, BUF ? 32 : 8>(a, bm, bn, wm, wn, li, lh, acc);
        ph.stored();
    } else {
        static_assert(EPI == 0 || (BM / WM) * (BN / WN) * 16 * (WN + 4) <= 2 * STAGE,
                      "staged epilogue needs 16 x (WN + 4) floats of LDS per wave");
        typename Staging<BUF, BM, BN, BK, NT, PADA, PADB, VEC, 4, 1, SWZ>::TC st4;
        st4.init(a, bm, bn);
        epilogue_mfma_staged<decltype(st4), MI, NI, WN>(a, st4, smem + wave * 16 * (WN + 4), wm, wn,
                                                         li, lh, lane, acc);
        ph.stored();
    }
}

// ---------------------------------------------------------------------------
// A tile kept in K order: As[BM][BK], each row one row of A.  Its BK / 4
// 16-byte chunks are permuted per row: chunk c of row m sits at chunk
// c ^ g(m), g(m) = (m / RP) % CPR, where CPR = BK / 4 chunks fill a row and
// RP = 16 / CPR rows fill the 256 bytes that span the 64 banks.  A load
// instruction fills 64 consecutive chunks (16 / CPR whole rows per 16-lane
// phase), and a fragment read takes one chunk of each of 16 consecutive
// rows; both then touch 16 different 16-byte bank groups.
// ---------------------------------------------------------------------------
template <int BK>
struct AKLayout {
    static_assert(BK == 16 || BK == 32 || BK == 64, "K-ordered A tile: BK in {16, 32, 64}");
    static constexpr int CPR = BK / 4;
    static constexpr int RP = 16 / CPR;
    static __device__ __forceinline__ int chunk_pos(int m, int c) { return c ^ ((m / RP) % CPR); }
};

// Buffer loads that write LDS directly: lane l's W floats land at
// lds + W * l, so one instruction fills 64 W consecutive floats of LDS, and
// a lane out of range writes zeros.  lds must be wave-uniform.
template <int W>
__device__ __forceinline__ void load_to_lds(rsrc_t r, float *lds, uint32_t voff) {
    static_assert(W == 1 || W == 4, "4 or 16 bytes per lane");
    typedef __attribute__((address_space(3))) void lds_t;
    if constexpr (W == 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_t *)lds, 16, voff, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_t *)lds, 4, voff, 0, 0, 0);
}

// The K-ordered A tile and the B tile ([BK][BN], unpadded) of one stage
// filled by loads that write LDS directly.  Instruction p of wave w fills
// floats (p * WAVES + w) * 64 W .. + 64 W of each tile, so each lane's
// global address is the one whose data belongs at its LDS position (for A
// through the chunk permutation of AKLayout).  Columns of A >= K and rows of
// B >= K read 0.0 (so do rows of A >= M); columns of B >= N read whatever
// lies there, which only reaches columns of C that are never stored.
template <int BM, int BN, int BK, int NT, int W>
struct DirectStage {
    static constexpr int WAVES = NT / 64;
    static constexpr int PER_INST = 64 * W;
    static_assert((BM * BK) % (NT * W) == 0 && (BK * BN) % (NT * W) == 0, "tiles must split into whole instructions");
    static constexpr int PA = BM * BK / (NT * W), PB = BK * BN / (NT * W);
    // With up to 8 instructions per tile the lanes' offsets are kept in
    // registers; with more (4-byte loads) they are recomputed at each load
    // from the lane index, which an empty asm makes opaque so that the
    // compiler cannot hoist PA + PB offsets into registers held across the
    // K loop (they would spill).
    static constexpr bool KEEP = PA + PB <= 8;
    rsrc_t ra;
    uint32_t aoff[KEEP ? PA : 1], boff[KEEP ? PB : 1];
    int acol[KEEP ? PA : 1];
    int wave, lane;
    int64_t lda, ldb;

    // row and column of A's tile held by instruction p at this lane
    __device__ __forceinline__ void a_pos(int p, int l, int &row, int &col) const {
        const int f = (p * WAVES + wave) * PER_INST + l * W;
        row = f / BK;
        const int pos = f % BK;
        col = 4 * AKLayout<BK>::chunk_pos(row, pos / 4) + pos % 4;
    }
    __device__ __forceinline__ uint32_t b_at(int p, int l) const {
        const int f = (p * WAVES + wave) * PER_INST + l * W;
        return (uint32_t)(((int64_t)(f / BN) * ldb + f % BN) * 4);
    }

    __device__ __forceinline__ void init(const Args &a, int bm, int tid) {
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        lane = tid & 63;
        lda = a.lda;
        ldb = a.ldb;
        ra = make_rsrc(a.A + (int64_t)bm * a.lda, ((int64_t)(a.M - bm - 1) * a.lda + a.K) * 4);
        if constexpr (KEEP) {
#pragma unroll
            for (int p = 0; p < PA; ++p) {
                int row, col;
                a_pos(p, lane, row, col);
                aoff[p] = (uint32_t)(((int64_t)row * a.lda + col) * 4);
                acol[p] = col;
            }
#pragma unroll
            for (int p = 0; p < PB; ++p) boff[p] = b_at(p, lane);
        }
    }

    // B rows k0.. from column bn, up to B's last element
    __device__ __forceinline__ rsrc_t b_rows(const Args &a, int bn, int k0) const {
        return make_rsrc(a.B + (int64_t)k0 * a.ldb + bn, ((int64_t)(a.K - k0 - 1) * a.ldb + (a.N - bn)) * 4);
    }

    __device__ __forceinline__ void load_a(const Args &a, float *As, int k0, int p) const {
        uint32_t off;
        int col;
        if constexpr (KEEP) {
            off = aoff[p];
            col = acol[p];
        } else {
            int l = lane, row;
            asm volatile("" : "+v"(l));
            a_pos(p, l, row, col);
            off = (uint32_t)(((int64_t)row * lda + col) * 4);
        }
        load_to_lds<W>(ra, As + (p * WAVES + wave) * PER_INST, k0 + col < a.K ? off + 4u * (uint32_t)k0 : kOutOfRange);
    }

    __device__ __forceinline__ void load_b(rsrc_t rb, float *Bs, int p) const {
        uint32_t off;
        if constexpr (KEEP) {
            off = boff[p];
        } else {
            int l = lane;
            asm volatile("" : "+v"(l));
            off = b_at(p, l);
        }
        load_to_lds<W>(rb, Bs + (p * WAVES + wave) * PER_INST, off);
    }

    // With K not a multiple of 4 (16-byte loads at 4-byte alignment), the
    // chunk of A that holds column K - 1 also brought columns K.. of its row
    // (the next row's first elements, or 0.0 past A's end).  B's rows >= K
    // read 0.0, but a non-finite value there would still make 0 * Inf = NaN,
    // so the stage's copies are cleared once the tile k0.. that holds column
    // K - 1 has landed, before the barrier that publishes it.
    __device__ __forceinline__ void fixup_a(const Args &a, float *As, int k0) const {
        static_assert(W == 4, "chunks of 4 columns");
#pragma unroll
        for (int p = 0; p < PA; ++p) {
            int col;
            if constexpr (KEEP) {
                col = acol[p];
            } else {
                int l = lane, row;
                asm volatile("" : "+v"(l));
                a_pos(p, l, row, col);
            }
            const int valid = a.K - (k0 + col);
            if (valid > 0 && valid < 4) {
                float *q = As + (p * WAVES + wave) * PER_INST + W * lane;
#pragma unroll
                for (int j = 1; j < 4; ++j)
                    if (j >= valid) q[j] = 0.0f;
            }
        }
    }
};

// One K tile of MFMAs over a K-ordered A tile.  Inside the tile the k index
// is permuted (the sum is the same in any order): of the wave's KX k values
// starting at k0, k-step j of lane half lh takes k = k0 + lh * KX / 2 + j, so
// lane (li, lh) reads A row (wm + 32 i + li) as KX / 8 chunks of 4
// consecutive k, one 128-bit read per chunk and block row i, and B row
// k0 + lh * KX / 2 + j.  a_row points at the lane's row of block row 0 in
// this stage, a_off[q] is 4 * (position of chunk q of its half); bp at B row
// k0 + lh * KX / 2, column wn + NI * li.  hook(j, u) as in mfma_tile.
// KX is the k extent the wave covers in this call (all of the tile, BK, or
// its wave group's share of it); A rows stay BK floats long.
// The operands of the last D k-steps' MFMAs of a K tile, held over to the
// next one (DF).
template <int MI, int NI, int D> struct KcPending {
    float x[D > 0 ? D : 1][MI];
    typename vec_t<NI>::type b[D > 0 ? D : 1];
};

// The MFMAs of the held-over k-steps STEPS - D .. STEPS - 1, in that order:
// an odd k-step into acc_odd when the odd k-steps have their own
// accumulators (CH == 2).
template <int MI, int NI, int CH, int D, int STEPS>
__device__ __forceinline__ void mfma_pending_kc(const KcPending<MI, NI, D> &pd, floatx16 (&acc)[MI][NI],
                                                floatx16 (&acc_odd)[MI][NI]) {
#pragma unroll
    for (int d = 0; d < D; ++d)
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int jj = 0; jj < NI; ++jj) {
                if (CH == 2 && ((STEPS - D + d) & 1))
                    acc_odd[i][jj] = __builtin_amdgcn_mfma_f32_32x32x2f32(pd.x[d][i], vget(pd.b[d], jj),
                                                                          acc_odd[i][jj], 0, 0, 0);
                else
                    acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x2f32(pd.x[d][i], vget(pd.b[d], jj), acc[i][jj],
                                                                      0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
}

// DF > 0: the last DF k-steps' MFMAs are not issued here but held in pd,
// and the caller issues them after the barrier that ends the tile (pd_in:
// this call issues the previous tile's, right after its own first fragment
// reads), so the matrix unit has work while those reads are in flight.
template <int BK, int MI, int NI, int SB, int FD, int CH, int RO, int PR, int KX, int DF, class Hook>
__device__ __forceinline__ void mfma_tile_kc(const float *a_row, const int (&a_off)[KX / 8], const float *bp,
                                             floatx16 (&acc)[MI][NI], floatx16 (&acc_odd)[MI][NI], Hook hook,
                                             KcPending<MI, NI, DF> &pd, bool pd_in) {
    typedef typename vec_t<NI>::type VB;
    static_assert(KX % 8 == 0 && KX <= BK, "k extent: whole chunks of 4 per lane half");
    constexpr int STEPS = KX / 2, QN = KX / 8;
    constexpr int RING = FD + 1;
    float4 av[2][MI];
    VB bv[RING];
    if (PR == 1) {
        __builtin_amdgcn_s_setprio(3);
        __builtin_amdgcn_sched_barrier(0);
    }
    // At the tile's start every wave of the workgroup reads LDS at once.
    // RO == 0: the first group of four k's of A, the B fragments and the
    // next group of A, all before the first MFMA.  RO == 1: the B fragment
    // first and the next group of A one k-step later, so the first MFMA
    // waits for about half as many bytes.  RO == 2: only the B fragment and
    // A block row 0 before the first MFMA, the rest of the group and the
    // next B fragment right after it.  Measured per block: RO == 1 is
    // 0.5-0.7% faster than RO == 0 on the 256 x 256 block and up to 4% on
    // 64 x 64 x 32, RO == 2 another 0.2-0.4% on 256 x 256 and 128 x 128 x 64;
    // both are 11% slower on 128 x 128 x 16 at four workgroups per CU where
    // the last round of tiles is partial (6144^3, 5120^3) and 0.4-1% slower
    // on 128 x 256 x 16 at 16384^2 x 128; no cause was found for those two.
    // PR == 1: the wave's issue priority falls from 3 to 0 over the K tile
    // (3 - 4q / QN at A group q), so of the waves on a SIMD the one furthest
    // behind in the tile issues first and they reach the closing barrier
    // closer together.  On the 256 x 256 x 32 block with 16 waves (four per
    // SIMD, one workgroup per CU) that is 0.1-0.6% faster in every one of 24
    // paired runs at 4096^3-16384^3, and faster than priority 3 for the first
    // quarter or half of the tile only.  On the 8-wave blocks with one
    // workgroup per CU it is slightly faster (128 x 128 x 64 and 128 x 256 x
    // 32: 0.15-0.7% in ten paired runs each, so those blocks use it too), and
    // up to 23% slower on blocks with two or four per CU where the last round
    // of tiles is partial.
    if (RO == 0) {
#pragma unroll
    for (int i = 0; i < MI; ++i) av[0][i] = *reinterpret_cast<const float4 *>(a_row + i * 32 * BK + a_off[0]);
#pragma unroll
    for (int f = 0; f < FD && f < STEPS; ++f) bv[f] = *reinterpret_cast<const VB *>(bp + f * SB);
    } else if (RO == 1) {
#pragma unroll
    for (int f = 0; f < FD && f < STEPS; ++f) bv[f] = *reinterpret_cast<const VB *>(bp + f * SB);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < MI; ++i) av[0][i] = *reinterpret_cast<const float4 *>(a_row + i * 32 * BK + a_off[0]);
    } else {
    bv[0] = *reinterpret_cast<const VB *>(bp);
    __builtin_amdgcn_sched_barrier(0);
    av[0][0] = *reinterpret_cast<const float4 *>(a_row + a_off[0]);
    }
    static_assert(DF >= 0 && DF <= STEPS, "held-over k-steps: at most a tile's");
    if (DF > 0 && pd_in) {
        __builtin_amdgcn_sched_barrier(0);
        mfma_pending_kc<MI, NI, CH, DF, STEPS>(pd, acc, acc_odd);
    }
    // RO == 2: the rest of the first group of A and the next B fragment
    // right after the first MFMA
    auto rest_of_first = [&]() {
#pragma unroll
        for (int i = 1; i < MI; ++i) av[0][i] = *reinterpret_cast<const float4 *>(a_row + i * 32 * BK + a_off[0]);
#pragma unroll
        for (int f = 1; f <= FD && f < STEPS; ++f) bv[f % RING] = *reinterpret_cast<const VB *>(bp + f * SB);
    };
#pragma unroll
    for (int q = 0; q < QN; ++q) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = 4 * q + e;
            if (PR == 1 && e == 0 && q > 0 && (4 * q) / QN != (4 * (q - 1)) / QN) {
                const int level = 3 - (4 * q) / QN;
                if (level == 2) __builtin_amdgcn_s_setprio(2);
                else if (level == 1) __builtin_amdgcn_s_setprio(1);
                else __builtin_amdgcn_s_setprio(0);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (RO == 0 && e == 0 && q + 1 < QN) {
#pragma unroll
                for (int i = 0; i < MI; ++i)
                    av[(q + 1) & 1][i] = *reinterpret_cast<const float4 *>(a_row + i * 32 * BK + a_off[q + 1]);
            }
            if (j + FD < STEPS && !(RO == 2 && j == 0))
                bv[(j + FD) % RING] = *reinterpret_cast<const VB *>(bp + (j + FD) * SB);
            if (RO >= 1 && e == 1 && q + 1 < QN) {
#pragma unroll
                for (int i = 0; i < MI; ++i)
                    av[(q + 1) & 1][i] = *reinterpret_cast<const float4 *>(a_row + i * 32 * BK + a_off[q + 1]);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (DF > 0 && j >= STEPS - DF) {
                const int d = j - (STEPS - DF);
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    const float4 &ac = av[q & 1][i];
                    pd.x[d][i] = e == 0 ? ac.x : e == 1 ? ac.y : e == 2 ? ac.z : ac.w;
                }
                pd.b[d] = bv[j % RING];
#pragma unroll
                for (int u = 0; u < MI * NI; ++u) hook(j, u);
                continue;
            }
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const float4 &ac = av[q & 1][i];
                const float x = e == 0 ? ac.x : e == 1 ? ac.y : e == 2 ? ac.z : ac.w;
#pragma unroll
                for (int jj = 0; jj < NI; ++jj) {
                    if (CH == 2 && (j & 1))
                        acc_odd[i][jj] = __builtin_amdgcn_mfma_f32_32x32x2f32(x, vget(bv[j % RING], jj),
                                                                              acc_odd[i][jj], 0, 0, 0);
                    else
                        acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x2f32(x, vget(bv[j % RING], jj),
                                                                          acc[i][jj], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    if (RO == 2 && j == 0 && i == 0 && jj == 0) {
                        rest_of_first();
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    hook(j, i * NI + jj);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }
}

// Epilogue of the K-ordered kernel: register r of block (mi, ni) on lane
// (li, lh) is tile row wm + 32 mi + 8 (r / 4) + 4 lh + r % 4, tile column
// wn + NI li + ni.
template <class TC, int MI, int NI, int GV = 32>
__device__ __forceinline__ void epilogue_mfma_kc(const Args &a, int bm, int bn, int wm, int wn, int li, int lh,
                                                 const floatx16 (&acc)[MI][NI]) {
    TC st;
    st.init(a, bm, bn);
    auto pos = [&](int v, int &r, int &c) {
        const int i = v / 16, reg = v % 16;
        r = wm + 32 * i + 8 * (reg >> 2) + 4 * lh + (reg & 3);
        c = wn + NI * li;
    };
    auto val = [&](int v, float (&x)[NI]) {
#pragma unroll
        for (int j = 0; j < NI; ++j) x[j] = acc[v / 16][j][v % 16];
    };
    epilogue<MI * 16, NI, TC, decltype(pos), decltype(val), GV>(a, st, pos, val);
}

// Epilogue of the K-ordered kernel with the old C values of its first NP
// vectors read ahead into pre (c_prefetch_kc, during the last K tile).
template <int MI, int NI>
__device__ __forceinline__ void kc_pos(int v, int wm, int wn, int li, int lh, int &r, int &c) {
    const int i = v / 16, reg = v % 16;
    r = wm + 32 * i + 8 * (reg >> 2) + 4 * lh + (reg & 3);
    c = wn + NI * li;
}

template <class TC, int MI, int NI, int NP>
__device__ __forceinline__ void c_prefetch_kc(const Args &a, int bm, int bn, int wm, int wn, int li, int lh,
                                              float (&pre)[NP][NI]) {
    if (a.beta == 0.0f) return;  // C is not read
    TC st;
    st.init(a, bm, bn);
#pragma unroll
    for (int v = 0; v < NP; ++v) {
        int r, c;
        kc_pos<MI, NI>(v, wm, wn, li, lh, r, c);
        st.load(a, r, c, pre[v]);
    }
}

template <class TC, int MI, int NI, int GV, int NP>
__device__ __forceinline__ void epilogue_mfma_kc_pre(const Args &a, int bm, int bn, int wm, int wn, int li,
                                                     int lh, const floatx16 (&acc)[MI][NI],
                                                     const float (&pre)[NP][NI]) {
    TC st;
    st.init(a, bm, bn);
    auto pos = [&](int v, int &r, int &c) { kc_pos<MI, NI>(v, wm, wn, li, lh, r, c); };
    auto val = [&](int v, float (&x)[NI]) {
#pragma unroll
        for (int j = 0; j < NI; ++j) x[j] = acc[v / 16][j][v % 16];
    };
    epilogue_pre<MI * 16, NI, TC, decltype(pos), decltype(val), GV, NP>(a, st, pos, val, pre);
}

// The barrier that ends a K tile of the LDS ring: this wave's loads but the
// newest N have landed (vmcnt; gfx9 encoding, vmcnt in bits 3:0 and 15:14,
// expcnt left at its maximum), its LDS reads have returned (lgkmcnt 0:
// nothing it read can be overwritten early), then every wave meets.
// __syncthreads() would wrap the barrier in workgroup fences, and those wait
// for every outstanding load that writes LDS, which would drain the ring; the
// empty asm statements and the scheduling fences keep the compiler from
// moving LDS accesses across the barrier instead.
template <int N>
__device__ __forceinline__ void ring_barrier() {
    static_assert(N >= 0 && N <= 63, "vmcnt is 6 bits");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------------------
// MFMA kernel with A kept in K order in LDS, both tiles loaded from global
// memory straight into LDS (16 bytes per lane when VEC == 4, else 4).  Same
// tiles and epilogue contract as sgemm_mfma; the SPLIT build also runs
// split-K and stream-K (phases 0-3 of Args).  RO is the order of the
// fragment reads at a K tile's start and PR the wave priority over a K tile
// (mfma_tile_kc).
//
// STG LDS stages form a ring ("如何高效实现矩阵乘", section "Double Buffer",
// with two; deeper rings for tiles whose arithmetic is too short to cover
// one load latency): the loads of K tile t + STG - 1 go, in pieces after the
// MFMAs of the first quarter of tile t's k-steps, into the stage tile t - 1
// was read from, and before the barrier that ends tile t each wave waits
// only until its loads of tile t + 1 have landed, leaving the later ones in
// flight.
//
// KG wave groups split every K tile: group g takes k in
// [g BK / KG, (g + 1) BK / KG) of each tile for the whole block tile, so a
// block tile that is the CU's only work still has KG waves per SIMD to
// interleave (in-workgroup split-K).  The groups' partial tiles are summed
// through LDS in group order (deterministic), and the epilogue is shared by
// every wave of the workgroup.
//
// UA: A and B loaded 16 bytes per lane at any 4-byte alignment (the range
// checks are per 4 bytes), the columns of A past K that a chunk brings along
// cleared in LDS once their tile has landed, C in 32-bit accesses.  DF: the
// last DF k-steps of MFMAs of each K tile are issued after the barrier that
// ends it (mfma_tile_kc).  CP: CP groups of the epilogue's old C values are
// read during the last K tile (one-group whole-tile builds).
// ---------------------------------------------------------------------------
template <int BM, int BN, int BK, int WM, int WN, int VEC, int WPE, bool SPLIT, int RO, int PR = 0,
          int KG = 1, int STG = 2, bool UA = false, int DF = 0, int CP = 0>
__global__ void __launch_bounds__(KG * (BM / WM) * (BN / WN) * 64)
__attribute__((amdgpu_waves_per_eu(WPE))) sgemm_mfma_kc(Args a) {
    constexpr int MI = WM / 32, NI = WN / 32;
    constexpr int WAVES_N = BN / WN;
    constexpr int WPG = (BM / WM) * WAVES_N;  // waves per group
    constexpr int NT = KG * WPG * 64;
    constexpr int SB = BN;
    constexpr int ASZ = BM * BK;
    constexpr int STAGE = ASZ + BK * SB;
    constexpr int KX = BK / KG;  // k per K tile of one group
    static_assert(MI == 1 || MI == 2 || MI == 4, "MI in {1, 2, 4}");
    static_assert(NI == 1 || NI == 2 || NI == 4, "NI in {1, 2, 4}");
    static_assert(KG == 1 || KG == 2 || KG == 4, "KG in {1, 2, 4}");
    static_assert(STG >= 2 && STG <= 4, "2 to 4 LDS stages");
    static_assert(!SPLIT || KG == 1, "split-K and stream-K builds run one wave group");
    // the groups' partial tiles, each in the lanes' own order
    constexpr int RED = KG > 1 ? KG * BM * BN : 0;
    constexpr int SMEM = STG * STAGE > RED ? STG * STAGE : RED;
    static_assert(!UA || (VEC == 4 && STG == 2), "rows at 4-byte alignment: 16-byte loads, two stages");
    static_assert(CP == 0 || (!SPLIT && KG == 1 && STG == 2), "C read ahead: one-group whole-tile builds");
    // CP groups of the epilogue's old C values are read during the last K tile
    constexpr int CPG = (UA ? 8 : 32) / NI > 0 ? (UA ? 8 : 32) / NI : 1;  // vectors per epilogue group
    constexpr int CPV = CP * (MI * 16 < CPG ? MI * 16 : CPG) < MI * 16 ? CP * (MI * 16 < CPG ? MI * 16 : CPG)
                                                                       : MI * 16;
    float cpre[CPV > 0 ? CPV : 1][NI];
    typedef DirectStage<BM, BN, BK, NT, VEC> D;
    // C in 32-bit accesses when the rows of C need not be 16-byte aligned
    typedef CStoreBuf<NI, UA ? 1 : VEC> TC;
    __shared__ __attribute__((aligned(16))) float smem[SMEM];

    PhaseLog ph;  // whole-tile builds only
    if (!SPLIT) ph.entry();
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int grp = wave / WPG, wg = wave % WPG;
    const int nbm = (a.M + BM - 1) / BM, nbn = (a.N + BN - 1) / BN;
    const int ntiles = nbm * nbn;
    const int wm = (wg / WAVES_N) * WM, wn = (wg % WAVES_N) * WN;
    const int li = lane & 31, lh = lane >> 5;
    const int KT_ALL = (a.K + BK - 1) / BK;

    constexpr int CH = MI * NI == 1 ? 2 : 1;
    floatx16 acc[MI][NI], acc_odd[MI][NI];

    // the lane's A row in a stage, its chunk positions, its B row and column
    constexpr int QN = KX / 8;
    const int a_row = (wm + li) * BK;
    int a_off[QN];
#pragma unroll
    for (int q = 0; q < QN; ++q) a_off[q] = 4 * AKLayout<BK>::chunk_pos(wm + li, (grp * KX) / 4 + lh * QN + q);
    const int b_off = ASZ + (grp * KX + lh * (KX / 2)) * SB + wn + NI * li;

    constexpr int STEPS = KX / 2;
    constexpr int LSTEPS = STEPS / 4 > 0 ? STEPS / 4 : 1;
    constexpr int NU = MI * NI;

    // acc = the product of the tile at (bm, bn) over K tiles [k_lo, k_hi)
    // (this wave group's share of each).  Starts and ends with every wave
    // past a barrier and every load landed, so it may run again on the same
    // LDS.
    auto k_range = [&](int bm, int bn, int k_lo, int k_hi) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = acc_odd[i][j][r] = 0.0f;
        const int KT = k_hi - k_lo, kb = k_lo * BK;
        // The loads of a K tile are spread over the MFMAs of the first
        // quarter of the k-steps (spreading them over a half or three
        // quarters measured the same).
        constexpr int DP = D::PA + D::PB;
        constexpr int DLPER = (DP + LSTEPS - 1) / LSTEPS;
        D d;
        d.init(a, bm, tid);
        // tiles 0 .. STG - 2 into stages 0 .. STG - 2
#pragma unroll
        for (int s = 0; s < STG - 1; ++s) {
            if (s < KT) {
                const rsrc_t rb = d.b_rows(a, bn, kb + s * BK);
#pragma unroll
                for (int p = 0; p < D::PA; ++p) d.load_a(a, smem + s * STAGE, kb + s * BK, p);
#pragma unroll
                for (int p = 0; p < D::PB; ++p) d.load_b(rb, smem + s * STAGE + ASZ, p);
            }
        }
        // this wave's loads of tile 0 have written LDS (a count beyond the
        // counter's 63 waits for a few loads more than needed)
        constexpr int AHEAD = (STG - 2) * DP < 63 ? (STG - 2) * DP : 63;
        if constexpr (STG == 2) {
            __builtin_amdgcn_s_waitcnt(0);
            if constexpr (UA)
                if ((a.K & 3) != 0 && kb < a.K && kb + BK > a.K) d.fixup_a(a, smem, kb);
            __syncthreads();
        } else if (KT >= STG - 1) {
            ring_barrier<AHEAD>();
        } else {
            ring_barrier<0>();
        }
        if (!SPLIT) ph.landed();
        // The stages as restrict pointers: the scoped no-alias information
        // lets the compiler see that the reads of the current stage need not
        // wait for the loads into another one (the waits are explicit).
        KcPending<MI, NI, DF> pd;
        auto tile_body = [&](const float *__restrict__ st, float *__restrict__ nx, int kn, bool issue,
                             bool pd_in) {
            const rsrc_t rb = d.b_rows(a, bn, kn);
            auto hook = [&](int j, int u) {
                if (j < LSTEPS && issue) {
#pragma unroll
                    for (int q = 0; q < DLPER; ++q) {
                        const int piece = j * DLPER + q;
                        if ((q * NU) / DLPER != u || piece >= DP) continue;
                        if (piece < D::PA) d.load_a(a, nx, kn, piece);
                        else d.load_b(rb, nx + ASZ, piece - D::PA);
                    }
                }
            };
            mfma_tile_kc<BK, MI, NI, SB, 1, CH, RO, PR, KX, DF>(st + a_row, a_off, st + b_off, acc, acc_odd,
                                                                hook, pd, pd_in);
        };
        if constexpr (STG == 2) {
            // the next tile is always loaded (past the last one it reads
            // zeros or the next range's data into a stage nobody reads)
            for (int t = 0; t < KT; ++t) {
                if (!SPLIT) ph.tile_begin();
                if constexpr (CP > 0) {
                    if (t == KT - 1) {
                        int li_ = li, lh_ = lh;
                        asm volatile("" : "+v"(li_), "+v"(lh_));
                        c_prefetch_kc<TC, MI, NI, CPV>(a, bm, bn, wm, wn, li_, lh_, cpre);
                    }
                }
                tile_body(smem + (t & 1) * STAGE, smem + ((t + 1) & 1) * STAGE, kb + (t + 1) * BK, true, t > 0);
                if (!SPLIT) ph.tile_mid();
                __builtin_amdgcn_s_waitcnt(0);
                if constexpr (UA) {
                    const int kn = kb + (t + 1) * BK;
                    if ((a.K & 3) != 0 && kn < a.K && kn + BK > a.K) d.fixup_a(a, smem + ((t + 1) & 1) * STAGE, kn);
                }
                __syncthreads();
                if (!SPLIT) ph.tile_end();
            }
        } else {
            int cur = 0, nxt = STG - 1;  // stage of tile t and of tile t + STG - 1
            for (int t = 0; t < KT; ++t) {
                const bool issue = t + STG - 1 < KT;
                if (!SPLIT) ph.tile_begin();
                tile_body(smem + cur * STAGE, smem + nxt * STAGE, kb + (t + STG - 1) * BK, issue, t > 0);
                if (!SPLIT) ph.tile_mid();
                // tile t + 1 has landed; tiles t + 2 .. t + STG - 1 may still be in flight
                if (issue)
                    ring_barrier<AHEAD>();
                else
                    ring_barrier<0>();
                if (!SPLIT) ph.tile_end();
                cur = cur + 1 == STG ? 0 : cur + 1;
                nxt = nxt + 1 == STG ? 0 : nxt + 1;
            }
        }
        // the last tile's held-over k-step
        if (DF > 0 && KT > 0) mfma_pending_kc<MI, NI, CH, DF, KX / 2>(pd, acc, acc_odd);
        if (CH == 2) {
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j) acc[i][j] += acc_odd[i][j];
        }
    };
    auto origin = [&](int tile, int &bm, int &bn) {
        int tm, tn;
        tile_of<2, 8>(tile, nbm, nbn, a.xcd_shift, tm, tn);
        bm = tm * BM;
        bn = tn * BN;
    };
    // In the split builds the epilogue sits in a loop (a stream-K worker may
    // finish a tile in either of its two K ranges), and its C offsets, which
    // depend only on the lane, would be hoisted out of that loop and held in
    // registers across the whole K loop.  The empty asm makes the lane's
    // coordinates opaque at each epilogue, so they are recomputed there.
    auto finish = [&](int bm, int bn) {
        int li_ = li, lh_ = lh;
        if constexpr (SPLIT) asm volatile("" : "+v"(li_), "+v"(lh_));
        if constexpr (CP > 0) {
            if (KT_ALL == 0) c_prefetch_kc<TC, MI, NI, CPV>(a, bm, bn, wm, wn, li_, lh_, cpre);  // no K loop ran
            epilogue_mfma_kc_pre<TC, MI, NI, UA ? 8 : 32, CPV>(a, bm, bn, wm, wn, li_, lh_, acc, cpre);
        }
        else
            epilogue_mfma_kc<TC, MI, NI, (SPLIT || UA) ? 8 : 32>(a, bm, bn, wm, wn, li_, lh_, acc);
    };

    if constexpr (!SPLIT && KG == 1) {
        int bm, bn;
        origin((int)blockIdx.x, bm, bn);
        k_range(bm, bn, 0, KT_ALL);
        ph.looped();
        finish(bm, bn);
        ph.stored();
    } else if constexpr (!SPLIT) {
        int bm, bn;
        origin((int)blockIdx.x, bm, bn);
        k_range(bm, bn, 0, KT_ALL);
        ph.looped();
        // Every wave is past the K loop's last barrier and every load has
        // landed: the stages are free.  Group g writes its partial tile to
        // region g in the lanes' own order: 4-float piece
        // ((i NI + j) 4 + q) WPG 64 + 64 wg + lane holds registers 4q .. 4q + 3
        // of block (i, j), so each write instruction of a wave fills 1 KiB of
        // consecutive LDS.
        constexpr int NTG = WPG * 64;  // threads per group
        float4 *red = reinterpret_cast<float4 *>(smem) + grp * (BM * BN / 4);
        const int tg = tid - grp * NTG;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int jj = 0; jj < NI; ++jj)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    red[((i * NI + jj) * 4 + q) * NTG + tg] =
                        make_float4(acc[i][jj][4 * q], acc[i][jj][4 * q + 1], acc[i][jj][4 * q + 2],
                                    acc[i][jj][4 * q + 3]);
        __syncthreads();
        // Thread t takes pieces f = t, t + NT, ...: the sum of the groups'
        // piece f, in group order.  Piece f holds 4 consecutive rows of one
        // column of C (registers 4q .. 4q + 3 of a block are rows
        // 8 q + 4 lh + 0 .. 3), stored one float at a time, 32 lanes to a
        // 128-byte row segment as in the one-group epilogue.
        constexpr int F4 = BM * BN / 4, PER = F4 / NT;
        static_assert(F4 % NT == 0, "the tile splits into whole 4-float pieces per thread");
        CStoreBuf<1, UA ? 1 : VEC> st;
        st.init(a, bm, bn);
        auto pos = [&](int v, int &r, int &c) {
            const int f = tid + NT * (v / 4), e = v % 4;
            const int blk = f / (4 * NTG), q = (f / NTG) % 4, t = f % NTG;
            const int i = blk / NI, jj = blk % NI, w = t / 64, l = t % 64;
            r = (w / WAVES_N) * WM + 32 * i + 8 * q + 4 * (l >> 5) + e;
            c = (w % WAVES_N) * WN + NI * (l & 31) + jj;
        };
        float4 sum[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const float4 *src = reinterpret_cast<const float4 *>(smem) + tid + NT * u;
            sum[u] = src[0];
#pragma unroll
            for (int g = 1; g < KG; ++g) {
                const float4 w = src[g * (BM * BN / 4)];
                sum[u].x += w.x;
                sum[u].y += w.y;
                sum[u].z += w.z;
                sum[u].w += w.w;
            }
        }
        auto val = [&](int v, float (&x)[1]) {
            const float4 &p4 = sum[v / 4];
            const int e = v % 4;
            x[0] = e == 0 ? p4.x : e == 1 ? p4.y : e == 2 ? p4.z : p4.w;
        };
        epilogue<4 * PER, 1, decltype(st), decltype(pos), decltype(val)>(a, st, pos, val);
        ph.stored();
    } else {
        // A partial tile in the lanes' own order (4-float chunks,
        // consecutive threads adjacent), written and added back.
        // Through a buffer descriptor over the one partial tile: the lane's
        // 32-bit offset is tid * 16 and each vector's constant part goes in
        // the scalar offset, so no 64-bit addresses are held.
        const uint32_t lane_off = (uint32_t)tid * 16u;
        auto store_partial = [&](float *dst) {
            const rsrc_t r = make_rsrc(dst, (int64_t)BM * BN * 4);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        f32x4 v;
                        v.x = acc[i][j][4 * q];
                        v.y = acc[i][j][4 * q + 1];
                        v.z = acc[i][j][4 * q + 2];
                        v.w = acc[i][j][4 * q + 3];
                        raw_store_v4f32(v, r, lane_off, (uint32_t)(((i * NI + j) * 4 + q) * NT * 16), 0);
                    }
        };
        // One accumulator block (16 values) in flight at a time: issued all
        // at once, the loads of a whole partial tile would hold as many
        // registers again as the accumulators and spill.
        auto add_partial = [&](const float *src) {
            const rsrc_t r = make_rsrc(src, (int64_t)BM * BN * 4);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j) {
                    f32x4 v[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        v[q] = raw_load_v4f32(r, lane_off, (uint32_t)(((i * NI + j) * 4 + q) * NT * 16), 0);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc[i][j][4 * q] += v[q].x;
                        acc[i][j][4 * q + 1] += v[q].y;
                        acc[i][j][4 * q + 2] += v[q].z;
                        acc[i][j][4 * q + 3] += v[q].w;
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
        };
        auto zero = [&]() {
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
        };
        // Stream-K: the K tiles of the last R tiles, R * KT_ALL in all, are
        // shared by S workers; worker w takes [w I / S, (w + 1) I / S), and
        // the worker holding K tile x of that sequence is owner(x).
        const int R = ntiles - a.sk_whole, S = a.sk_workers;
        const int64_t I = (int64_t)R * KT_ALL;
        auto first = [&](int64_t w) { return w * I / S; };
        auto owner = [&](int64_t x) { return (int)(((x + 1) * S - 1) / I); };
        int bm, bn;
        if (a.phase == 1 || a.phase == 3) {
            // The partials of one tile summed in a fixed order, then C:
            // split-K in split order, stream-K in worker order.
            zero();
            if (a.phase == 1) {
                const int tile = (int)blockIdx.x;
                origin(tile, bm, bn);
                for (int sp = 0; sp < a.splits; ++sp)
                    add_partial(a.partial + ((int64_t)tile * a.splits + sp) * (BM * BN));
            } else {
                const int r = (int)blockIdx.x;
                const int w0 = owner((int64_t)r * KT_ALL), w1 = owner((int64_t)(r + 1) * KT_ALL - 1);
                if (w0 == w1) return;  // one worker held the tile whole: already in C
                origin(a.sk_whole + r, bm, bn);
                for (int w = w0; w <= w1; ++w) {
                    if (first(w) == first(w + 1)) continue;  // a worker with no K tiles
                    add_partial(a.partial + ((int64_t)w * 2 + (first(w) / KT_ALL == r ? 0 : 1)) * (BM * BN));
                }
            }
            finish(bm, bn);
            return;
        }
        // Phases 0 and 2: one or two K ranges, each stored as a partial tile
        // or, when it is a whole tile, finished into C.
        //   split-K: this split's K range of its tile;
        //   stream-K: a whole tile (the first sk_whole workgroups), or a
        //   worker's K tiles, fewer than KT_ALL (R < S), so at most the end
        //   of one tile (slot 0) and the start of the next (slot 1).
        const bool worker = a.phase == 2 && (int)blockIdx.x >= a.sk_whole;
        const int w = (int)blockIdx.x - a.sk_whole;
        int64_t x = worker ? first(w) : 0;
        const int64_t end = worker ? first(w + 1) : 0;
#pragma unroll 1
        for (int slot = 0; slot < 2; ++slot) {
            int tile, k_lo, k_hi;
            float *dst = nullptr;
            if (a.phase == 0) {
                if (slot > 0) break;
                const int split = (int)blockIdx.x / ntiles;
                tile = (int)blockIdx.x - split * ntiles;
                k_lo = (int)((int64_t)KT_ALL * split / a.splits);
                k_hi = (int)((int64_t)KT_ALL * (split + 1) / a.splits);
                dst = a.partial + ((int64_t)tile * a.splits + split) * (BM * BN);
            } else if (!worker) {
                if (slot > 0) break;
                tile = (int)blockIdx.x;
                k_lo = 0;
                k_hi = KT_ALL;
            } else {
                if (x >= end) break;
                const int r = (int)(x / KT_ALL);
                tile = a.sk_whole + r;
                k_lo = (int)(x - (int64_t)r * KT_ALL);
                k_hi = end - x < KT_ALL - k_lo ? k_lo + (int)(end - x) : KT_ALL;
                if (k_lo != 0 || k_hi != KT_ALL) dst = a.partial + ((int64_t)w * 2 + slot) * (BM * BN);
                x += k_hi - k_lo;
            }
            origin(tile, bm, bn);
            k_range(bm, bn, k_lo, k_hi);
            if (dst)
                store_partial(dst);
            else
                finish(bm, bn);
        }
    }
}

}  // namespace sgk
