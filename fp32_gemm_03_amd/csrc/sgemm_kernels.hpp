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
//   1. global -> VGPR: A's BM x BK block and B's BK x BN block.  Elements
//      outside M, N or K load as 0.0 (zero padding of partial tiles, "3.3
//      Shared memory ו tiling תרגול", exercise 1).  B is read with 128-bit
//      loads along N when VEC == 4, else with 32-bit loads.  A is read as
//      4 rows x 1 column per thread group: consecutive lanes walk K, so every
//      load instruction covers whole row segments of A.
//   2. VGPR -> LDS: A is stored TRANSPOSED (k-major, As[k][m]) with its rows
//      padded by PADA floats, one 128-bit store per 4 rows; B is stored as it
//      is (Bs[k][n], padded by PADB).  This is the layout of "SGEMM CUDA kernel
//      (Second Half)", Part 8 "Transposed As": A read as 4 x 1, written as a
//      1 x 4 vector into a transposed tile whose rows are shifted by 4 extra
//      columns so that the vector stores do not collide in LDS banks.
//   3. Two LDS stages: the global loads of step t+1 are issued before the
//      LDS reads and arithmetic of step t, and written to the other stage
//      afterwards; one workgroup barrier per step ("如何高效实现矩阵乘", section
//      "Double Buffer").
//
// Workgroup -> tile order: consecutive workgroup ids walk one row of C tiles
// (the M tile index is the slow one), "如何高效实现矩阵乘", section "Wave & L2
// cache Hit Rate".
//
// Nothing here includes or calls the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
    // Nonzero when every byte offset the fast path forms inside one block
    // tile fits in 31 bits (set by the host per variant).
    int fast;
};

typedef float floatx16 __attribute__((ext_vector_type(16)));

template <int W> struct vec_t;
template <> struct vec_t<1> { typedef float type; };
template <> struct vec_t<2> { typedef float2 type; };
template <> struct vec_t<4> { typedef float4 type; };

__device__ __forceinline__ float vget(float v, int) { return v; }
__device__ __forceinline__ float vget(const float2 &v, int i) { return i == 0 ? v.x : v.y; }
__device__ __forceinline__ float vget(const float4 &v, int i) {
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

template <class T>
__device__ __forceinline__ T load_at(const char *base, uint32_t byte_off) {
    return *reinterpret_cast<const T *>(base + byte_off);
}

// ---------------------------------------------------------------------------
// A tile: BM x BK block of A -> As[BK][BM + PADA] (transposed).
// Thread tid covers column tid % BK of rows r0 + {0..3} + p * ROWS_PER_PASS,
// r0 = 4 * (tid / BK): a load instruction reads NT/BK row segments of BK
// consecutive floats, and each thread writes one 128-bit vector per 4 rows.
//
// load_fast: the block lies inside M and the K tile is full, so nothing is
// checked; the address is a uniform (scalar) tile base plus a 32-bit
// per-thread offset.  load_checked: every element is checked against M and K
// and loads 0.0 outside.
// ---------------------------------------------------------------------------
template <int BM, int BK, int NT, int PADA>
struct ATile {
    static_assert(BM % 4 == 0, "BM must be a multiple of 4");
    static_assert(NT % BK == 0, "BK must divide the thread count");
    static constexpr int ROWS_PER_PASS = 4 * (NT / BK);
    static_assert(BM % ROWS_PER_PASS == 0, "A tile must divide evenly over the threads");
    static constexpr int PER = BM / ROWS_PER_PASS;
    static constexpr int SA = BM + PADA;

    float4 reg[PER];
    int col;           // column inside the tile
    int r0;            // first row inside the block
    uint32_t off[4];   // fast path: ((r0 + c) * lda + col) * 4

    __device__ __forceinline__ void init(const Args &a, int tid) {
        col = tid % BK;
        r0 = 4 * (tid / BK);
#pragma unroll
        for (int c = 0; c < 4; ++c) off[c] = (uint32_t)(((int64_t)(r0 + c) * a.lda + col) * 4);
    }

    // tile: byte address of A[bm][k0]; pass: ROWS_PER_PASS * lda * 4
    __device__ __forceinline__ void load_fast(const char *tile, int64_t pass) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const char *sb = tile + p * pass;
            reg[p].x = load_at<float>(sb, off[0]);
            reg[p].y = load_at<float>(sb, off[1]);
            reg[p].z = load_at<float>(sb, off[2]);
            reg[p].w = load_at<float>(sb, off[3]);
        }
    }

    __device__ __forceinline__ void load_checked(const Args &a, int bm, int k0) {
        const bool kin = (k0 + col) < a.K;
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int row = bm + r0 + p * ROWS_PER_PASS;
            const float *q = a.A + (int64_t)row * a.lda + k0 + col;
            const int rl = a.M - row;
            reg[p].x = (kin && rl > 0) ? q[0] : 0.0f;
            reg[p].y = (kin && rl > 1) ? q[a.lda] : 0.0f;
            reg[p].z = (kin && rl > 2) ? q[2 * a.lda] : 0.0f;
            reg[p].w = (kin && rl > 3) ? q[3 * a.lda] : 0.0f;
        }
    }

    __device__ __forceinline__ void store(float *As, int tid) const {
        float *dst = As + (tid % BK) * SA + 4 * (tid / BK);
#pragma unroll
        for (int p = 0; p < PER; ++p)
            *reinterpret_cast<float4 *>(dst + p * ROWS_PER_PASS) = reg[p];
    }
};

// ---------------------------------------------------------------------------
// B tile: BK x BN block of B -> Bs[BK][BN + PADB] (as is), VEC floats per
// load.  Consecutive threads take consecutive VEC-wide pieces of a row.
// ---------------------------------------------------------------------------
template <int BN, int BK, int NT, int PADB, int VEC>
struct BTile {
    static constexpr int PER_ROW = BN / VEC;  // pieces per tile row
    static_assert(BN % VEC == 0, "BN must be a multiple of VEC");
    static_assert(NT % PER_ROW == 0 || PER_ROW % NT == 0, "B tile rows and threads must nest");
    static constexpr int ITEMS = BK * PER_ROW;
    static_assert(ITEMS % NT == 0, "B tile must divide evenly over the threads");
    static constexpr int PER = ITEMS / NT;
    static constexpr int SB = BN + PADB;
    typedef typename vec_t<VEC>::type V;

    V reg[PER];
    int k_first;   // tile row of piece 0
    int n_first;   // column of piece 0 inside the tile
    uint32_t off;  // fast path: (k_first * ldb + n_first) * 4

    // piece p of a thread: tile row k_first + dk(p), tile column n_first + dn(p)
    static __device__ __forceinline__ constexpr int dk(int p) {
        return NT % PER_ROW == 0 ? p * (NT / PER_ROW) : (p * NT) / PER_ROW;
    }
    static __device__ __forceinline__ constexpr int dn(int p) {
        return NT % PER_ROW == 0 ? 0 : ((p * NT) % PER_ROW) * VEC;
    }

    __device__ __forceinline__ void init(const Args &a, int tid) {
        k_first = tid / PER_ROW;
        n_first = (tid % PER_ROW) * VEC;
        off = (uint32_t)(((int64_t)k_first * a.ldb + n_first) * 4);
    }

    // tile: byte address of B[k0][bn]; ldb_bytes: ldb * 4
    __device__ __forceinline__ void load_fast(const char *tile, int64_t ldb_bytes) {
#pragma unroll
        for (int p = 0; p < PER; ++p)
            reg[p] = load_at<V>(tile + dk(p) * ldb_bytes + dn(p) * 4, off);
    }

    __device__ __forceinline__ void load_checked(const Args &a, int bn, int k0) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int n = bn + n_first + dn(p);
            const int k = k0 + k_first + dk(p);
            // VEC == 4 only when N % 4 == 0: a piece is all in or all out
            if (n < a.N && k < a.K)
                reg[p] = *reinterpret_cast<const V *>(a.B + (int64_t)k * a.ldb + n);
            else
                reg[p] = V{};
        }
    }

    __device__ __forceinline__ void store(float *Bs, int tid) const {
        float *dst = Bs + (tid / PER_ROW) * SB + (tid % PER_ROW) * VEC;
#pragma unroll
        for (int p = 0; p < PER; ++p)
            *reinterpret_cast<V *>(dst + dk(p) * SB + dn(p)) = reg[p];
    }
};

// Loads of K tile t into the staging registers: the fast path for a block
// inside M and N with a full K tile, the checked path otherwise.
template <class TA, class TB, int BK>
__device__ __forceinline__ void load_tile(const Args &a, TA &ta, TB &tb, bool interior, int bm,
                                          int bn, int t) {
    const int k0 = t * BK;
    if (interior && k0 + BK <= a.K) {
        const char *at = reinterpret_cast<const char *>(a.A + (int64_t)bm * a.lda + k0);
        const char *bt = reinterpret_cast<const char *>(a.B + (int64_t)k0 * a.ldb + bn);
        ta.load_fast(at, (int64_t)TA::ROWS_PER_PASS * a.lda * 4);
        tb.load_fast(bt, a.ldb * 4);
    } else {
        ta.load_checked(a, bm, k0);
        tb.load_checked(a, bn, k0);
    }
}

// Epilogue store of W consecutive columns: C = alpha*acc + beta*C (C read only
// when beta != 0).  CHECK masks rows and columns to the matrix.  VEC == 4
// means N, ldc and C are 16-byte friendly, so a W-wide group at a multiple of
// W is all in or all out and goes out as one vector store.
template <int W, int VEC, bool CHECK>
__device__ __forceinline__ void store_c(const Args &a, int row, int col, const float (&v)[W]) {
    if (CHECK && row >= a.M) return;
    float *c = a.C + (int64_t)row * a.ldc + col;
    if (VEC == 4 && W > 1) {
        if (CHECK && col >= a.N) return;
        typedef typename vec_t<W>::type V;
        V out;
        float *o = reinterpret_cast<float *>(&out);
        if (a.beta != 0.0f) {
            const V old = *reinterpret_cast<const V *>(c);
#pragma unroll
            for (int i = 0; i < W; ++i) o[i] = fmaf(a.alpha, v[i], a.beta * vget(old, i));
        } else {
#pragma unroll
            for (int i = 0; i < W; ++i) o[i] = a.alpha * v[i];
        }
        *reinterpret_cast<V *>(c) = out;
    } else {
#pragma unroll
        for (int i = 0; i < W; ++i) {
            if (!CHECK || col + i < a.N) {
                const float r = a.beta != 0.0f ? fmaf(a.alpha, v[i], a.beta * c[i]) : a.alpha * v[i];
                c[i] = r;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// VALU kernel.  Block tile BM x BN, NT = (BM / (8*TM)) * (BN / (8*TN)) * 64.
// A wave owns an (8*TM) x (8*TN) tile; lane (ly, lx) = (lane / 8, lane % 8)
// owns rows  wm + 4*ly + {0..3} + 32*s  (s < TM/4)  and
//      cols  wn + 4*lx + {0..3} + 32*s  (s < TN/4),
// so every LDS read is one 128-bit load that 8 lanes share (broadcast).
// ---------------------------------------------------------------------------
template <int BM, int BN, int BK, int TM, int TN, int PADA, int PADB, int VEC, bool CHECK>
__device__ __forceinline__ void valu_epilogue(const Args &a, int bm, int bn, int wm, int wn,
                                              int ly, int lx, const float (&acc)[TM][TN]) {
    // 8 lanes with the same ly cover 32 consecutive columns (128 bytes) of a row
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int row = bm + wm + 4 * ly + (i & 3) + 32 * (i >> 2);
#pragma unroll
        for (int s = 0; s < TN / 4; ++s) {
            const int col = bn + wn + 4 * lx + 32 * s;
            float v[4] = {acc[i][4 * s], acc[i][4 * s + 1], acc[i][4 * s + 2], acc[i][4 * s + 3]};
            store_c<4, VEC, CHECK>(a, row, col, v);
        }
    }
}

template <int BM, int BN, int BK, int TM, int TN, int PADA, int PADB, int VEC, int WPE>
__global__ void __launch_bounds__((BM / (8 * TM)) * (BN / (8 * TN)) * 64)
__attribute__((amdgpu_waves_per_eu(WPE))) sgemm_valu(Args a) {
    constexpr int WM = 8 * TM, WN = 8 * TN;
    constexpr int WAVES_N = BN / WN;
    constexpr int NT = (BM / WM) * WAVES_N * 64;
    static_assert(TM % 4 == 0 && TN % 4 == 0, "micro-tile sides must be multiples of 4");
    constexpr int SA = BM + PADA, SB = BN + PADB;
    constexpr int STAGE = BK * (SA + SB);
    __shared__ __attribute__((aligned(16))) float smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int nbn = (a.N + BN - 1) / BN;
    const int bm = (int)(blockIdx.x / nbn) * BM;
    const int bn = (int)(blockIdx.x % nbn) * BN;
    const int wm = (wave / WAVES_N) * WM, wn = (wave % WAVES_N) * WN;
    const int ly = lane >> 3, lx = lane & 7;
    const bool interior = a.fast && bm + BM <= a.M && bn + BN <= a.N;

    ATile<BM, BK, NT, PADA> ta;
    BTile<BN, BK, NT, PADB, VEC> tb;
    ta.init(a, tid);
    tb.init(a, tid);

    float acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = 0.0f;

    const int KT = (a.K + BK - 1) / BK;
    if (KT > 0) {
        load_tile<decltype(ta), decltype(tb), BK>(a, ta, tb, interior, bm, bn, 0);
        ta.store(smem, tid);
        tb.store(smem + BK * SA, tid);
    }
    __syncthreads();

    for (int t = 0; t < KT; ++t) {
        const float *As = smem + (t & 1) * STAGE;
        const float *Bs = As + BK * SA;
        if (t + 1 < KT) load_tile<decltype(ta), decltype(tb), BK>(a, ta, tb, interior, bm, bn, t + 1);
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
            ta.store(An, tid);
            tb.store(An + BK * SA, tid);
        }
        __syncthreads();
    }

    if (bm + BM <= a.M && bn + BN <= a.N)
        valu_epilogue<BM, BN, BK, TM, TN, PADA, PADB, VEC, false>(a, bm, bn, wm, wn, ly, lx, acc);
    else
        valu_epilogue<BM, BN, BK, TM, TN, PADA, PADB, VEC, true>(a, bm, bn, wm, wn, ly, lx, acc);
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
template <int BM, int BN, int WM, int WN, int VEC, bool CHECK>
__device__ __forceinline__ void mfma_epilogue(const Args &a, int bm, int bn, int wm, int wn,
                                              int li, int lh,
                                              const floatx16 (&acc)[WM / 32][WN / 32]) {
    constexpr int MI = WM / 32, NI = WN / 32;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int ib = 8 * (r >> 2) + 4 * lh + (r & 3);
            const int row = bm + wm + MI * ib + i;
            const int col = bn + wn + NI * li;
            float v[NI];
#pragma unroll
            for (int j = 0; j < NI; ++j) v[j] = acc[i][j][r];
            store_c<NI, VEC, CHECK>(a, row, col, v);
        }
    }
}

template <int BM, int BN, int BK, int WM, int WN, int PADA, int PADB, int VEC, int WPE>
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
    typedef typename vec_t<MI>::type VA;
    typedef typename vec_t<NI>::type VB;
    __shared__ __attribute__((aligned(16))) float smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int nbn = (a.N + BN - 1) / BN;
    const int bm = (int)(blockIdx.x / nbn) * BM;
    const int bn = (int)(blockIdx.x % nbn) * BN;
    const int wm = (wave / WAVES_N) * WM, wn = (wave % WAVES_N) * WN;
    const int li = lane & 31, lh = lane >> 5;
    const bool interior = a.fast && bm + BM <= a.M && bn + BN <= a.N;

    ATile<BM, BK, NT, PADA> ta;
    BTile<BN, BK, NT, PADB, VEC> tb;
    ta.init(a, tid);
    tb.init(a, tid);

    floatx16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int KT = (a.K + BK - 1) / BK;
    if (KT > 0) {
        load_tile<decltype(ta), decltype(tb), BK>(a, ta, tb, interior, bm, bn, 0);
        ta.store(smem, tid);
        tb.store(smem + BK * SA, tid);
    }
    __syncthreads();

    for (int t = 0; t < KT; ++t) {
        const float *As = smem + (t & 1) * STAGE;
        const float *Bs = As + BK * SA;
        if (t + 1 < KT) load_tile<decltype(ta), decltype(tb), BK>(a, ta, tb, interior, bm, bn, t + 1);
        const float *ap = As + lh * SA + wm + MI * li;
        const float *bp = Bs + lh * SB + wn + NI * li;
        VA av[2];
        VB bv[2];
        av[0] = *reinterpret_cast<const VA *>(ap);
        bv[0] = *reinterpret_cast<const VB *>(bp);
#pragma unroll
        for (int k = 0; k < BK; k += 2) {
            const int cur = (k >> 1) & 1;
            if (k + 2 < BK) {
                av[cur ^ 1] = *reinterpret_cast<const VA *>(ap + (k + 2) * SA);
                bv[cur ^ 1] = *reinterpret_cast<const VB *>(bp + (k + 2) * SB);
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(vget(av[cur], i), vget(bv[cur], j),
                                                                     acc[i][j], 0, 0, 0);
        }
        if (t + 1 < KT) {
            float *An = smem + ((t + 1) & 1) * STAGE;
            ta.store(An, tid);
            tb.store(An + BK * SA, tid);
        }
        __syncthreads();
    }

    if (bm + BM <= a.M && bn + BN <= a.N)
        mfma_epilogue<BM, BN, WM, WN, VEC, false>(a, bm, bn, wm, wn, li, lh, acc);
    else
        mfma_epilogue<BM, BN, WM, WN, VEC, true>(a, bm, bn, wm, wn, li, lh, acc);
}

}  // namespace sgk
