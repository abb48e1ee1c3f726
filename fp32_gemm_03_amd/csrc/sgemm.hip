// sgemm.hip -- C ABI of the gfx950 FP32 SGEMM library (see include/sgemm.h):
// argument checks, the table of compiled kernel variants, the shape-based
// choice of variant, and the launch on the caller's stream.
//
// The only state is a per-device cache of the machine shape (compute units
// and XCDs), read once.  Every call validates, picks a variant and enqueues
// one kernel (two for split-K and stream-K: the partial tiles, then their sum
// in a fixed order).  Nothing here allocates device memory; split-K writes
// its partial tiles to a workspace the caller owns.
#include "sgemm.h"

#include <limits.h>
#include <stdint.h>

#include <mutex>

#include "sgemm_kernels.hpp"

namespace {

using sgk::Args;

typedef void (*KernelFn)(Args);

struct Variant {
    const char *name;
    int path;           // SGEMM_PATH_VALU or SGEMM_PATH_MFMA
    int bm, bn, bk;     // block tile
    int threads;        // workgroup size
    KernelFn vec4;      // buffer accesses; B, C and their leading dimensions 16-byte friendly
    KernelFn vec1;      // buffer accesses, 32-bit
    KernelFn generic;   // per-element checked pointer accesses (any leading dimension)
    KernelFn split4;    // split-K and stream-K, as vec4 (nullptr: no split-K build of this variant)
    int a128;           // 1: the vec4 build also reads A 128 bits at a time along K
    int streamk;        // 1: the split builds also run stream-K (phases 2 and 3)
    int generic_buf;    // 1: `generic` is a buffer-access build too (no plain-pointer
                        // build exists), so it needs in-tile offsets below 2^31
    KernelFn vec4u;     // 16-byte loads of A and B at any 4-byte alignment, 32-bit C
                        // (nullptr: no such build)
    KernelFn split4u;   // split-K (and stream-K), as vec4u
};

// VALU: BM x BN x BK block, waves of (8 TM) x (8 TN), TM x TN per lane.
#define VALU_CFG(BM, BN, BK, TM, TN, PA, PB, WPE)                                       \
    {"valu_" #BM "x" #BN "x" #BK "_t" #TM "x" #TN, SGEMM_PATH_VALU, BM, BN, BK,           \
     (BM / (8 * TM)) * (BN / (8 * TN)) * 64,                                             \
     sgk::sgemm_valu<BM, BN, BK, TM, TN, PA, PB, 4, WPE, true>,                       \
     sgk::sgemm_valu<BM, BN, BK, TM, TN, PA, PB, 1, WPE, true>,                       \
     sgk::sgemm_valu<BM, BN, BK, TM, TN, PA, PB, 1, WPE, false>, nullptr, 0, 0}

// A register-staged MFMA block (sgemm_mfma), A transposed in LDS: padded by
// PA, or unpadded and XOR-swizzled (SWZ); EPI 1 stages the epilogue through
// LDS; ORD is the workgroup -> tile order.
#define MFMA_CFG(BM, BN, BK, WM, WN, PA, WPE, ORD, EPI, SWZ, SUFFIX)                     \
    {"mfma_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN SUFFIX, SGEMM_PATH_MFMA, BM, BN, BK,    \
     (BM / WM) * (BN / WN) * 64,                                                         \
     sgk::sgemm_mfma<BM, BN, BK, WM, WN, PA, 0, 4, WPE, true, 1, ORD, EPI, SWZ, false>,  \
     sgk::sgemm_mfma<BM, BN, BK, WM, WN, PA, 0, 1, WPE, true, 1, ORD, EPI, SWZ, false>,  \
     sgk::sgemm_mfma<BM, BN, BK, WM, WN, PA, 0, 1, WPE, false, 1, ORD, EPI, SWZ, false>, \
     nullptr, 0, 0}

// A variant with A kept in K order (sgemm_mfma_kc): its 128-bit builds, and
// its builds for rows at 4-byte alignment (16-byte loads of A and B, 32-bit
// C), load straight into LDS, as whole tiles and with split-K and stream-K.
// Its 32-bit and checked whole-tile builds are the same block on the
// interleaved schedule (A transposed, padded by PA or XOR-swizzled):
// loading straight into LDS 4 bytes per lane is 4% slower than that at
// 8191^3 (140 against 145-146 TFLOP/s).  Those two sum the k of a K tile in
// the same order as each other, the 16-byte load builds in another.  RO is
// the order of the LDS fragment reads at a K tile's start (mfma_tile_kc),
// chosen per block by measurement.  Every build maps workgroups to tiles
// with tile_of<2, 8> (each XCD on its own tile columns), and holds each K
// tile's last k-step of MFMAs over the barrier (DF: 0.2-7% faster on most
// blocks and shapes, 9% on 256 x 256 x 4096 in 16 parts, at most 1.5%
// slower on a few).  The split builds of the 64 x 64 blocks hold the last
// two k-steps (SD 2: another 2-4% on their split-K and stream-K shapes; level
// on the larger blocks' split builds, mixed on whole tiles).  CPG groups of
// the epilogue's old C values are read during the last K tile (the 128 x 256
// x 16 block of low K: 118.3 against 116.3 TFLOP/s at 16384^2 x 128 with
// beta = 1; slower on the 64 x 64 x 32 block, level with beta = 0).
#define MFMA_CFG_KCD(BM, BN, BK, WM, WN, WPE, PA, SWZ, RO, SD, CPG, SUFFIX)             \
    {"mfma_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN SUFFIX, SGEMM_PATH_MFMA, BM, BN, BK,    \
     (BM / WM) * (BN / WN) * 64,                                                         \
     sgk::sgemm_mfma_kc<BM, BN, BK, WM, WN, 4, WPE, false, RO, 0, 1, 2, false, 1, CPG>, \
     sgk::sgemm_mfma<BM, BN, BK, WM, WN, PA, 0, 1, WPE, true, 1, 2, 0, SWZ, true>,       \
     sgk::sgemm_mfma<BM, BN, BK, WM, WN, PA, 0, 1, WPE, false, 1, 2, 0, SWZ, true>,      \
     sgk::sgemm_mfma_kc<BM, BN, BK, WM, WN, 4, WPE, true, RO, 0, 1, 2, false, SD>, 1, 1, 0, \
     sgk::sgemm_mfma_kc<BM, BN, BK, WM, WN, 4, WPE, false, RO, 0, 1, 2, true, 1, CPG>,  \
     sgk::sgemm_mfma_kc<BM, BN, BK, WM, WN, 4, WPE, true, RO, 0, 1, 2, true, SD>}

// A small K-ordered block of 32 x 32 waves split over KG wave groups; all
// four builds are sgemm_mfma_kc (128-bit, 4-byte loads into LDS twice, and
// 16-byte loads at 4-byte alignment), so even its checked build needs
// in-tile offsets below 2^31.
#define MFMA_CFG_KG(BM, BN, BK, KG, RO, SUFFIX)                                               \
    {"mfma_" #BM "x" #BN "x" #BK "_w32x32" SUFFIX, SGEMM_PATH_MFMA, BM, BN, BK,                 \
     KG * (BM / 32) * (BN / 32) * 64,                                                         \
     sgk::sgemm_mfma_kc<BM, BN, BK, 32, 32, 4, 4, false, RO, 0, KG, 2, false, 1>,          \
     sgk::sgemm_mfma_kc<BM, BN, BK, 32, 32, 1, 4, false, RO, 0, KG, 2, false, 1>,          \
     sgk::sgemm_mfma_kc<BM, BN, BK, 32, 32, 1, 4, false, RO, 0, KG, 2, false, 1>, nullptr, 1, 0, 1, \
     sgk::sgemm_mfma_kc<BM, BN, BK, 32, 32, 4, 4, false, RO, 0, KG, 2, true, 1>}

// The table holds the blocks the choice by shape can pick (the VALU pair and
// the K-ordered blocks) and the alternatives kept for measurement: the
// XCD-grouped tile order, the LDS-staged epilogue and A unpadded with an XOR
// swizzle, each on the register-staged 128 x 256 / 256 x 128 x 16 blocks,
// and a four-stage LDS ring on the 256 x 256 block.
const Variant kVariants[] = {
    VALU_CFG(128, 128, 16, 8, 8, 4, 0, 4),                         // 0: 8 x 8 per lane
    VALU_CFG(128, 256, 16, 8, 16, 4, 0, 2),                        // 1: 8 x 16 per lane
    MFMA_CFG(128, 256, 16, 64, 128, 4, 2, 1, 0, false, "_xcd"),    // 2: XCD-grouped tile order
    MFMA_CFG(256, 128, 16, 128, 64, 4, 2, 1, 0, false, "_xcd"),    // 3: XCD-grouped tile order
    MFMA_CFG(128, 256, 16, 64, 128, 4, 2, 0, 1, false, "_ldsepi"), // 4: LDS-staged epilogue
    MFMA_CFG(256, 128, 16, 128, 64, 4, 2, 0, 1, false, "_ldsepi"), // 5: LDS-staged epilogue
    MFMA_CFG(128, 256, 16, 64, 128, 0, 2, 0, 0, true, "_xorA"),    // 6: A unpadded, XOR-swizzled
    MFMA_CFG_KCD(256, 256, 32, 128, 64, 2, 4, false, 2, 1, 0, "_kcd"),    // 7: 8 waves, 2 per SIMD
    MFMA_CFG_KCD(128, 128, 16, 64, 64, 4, 4, false, 0, 1, 0, "_wpe4_kcd"),  // 8: 4 workgroups per CU
    MFMA_CFG_KCD(128, 256, 16, 64, 128, 2, 0, true, 0, 1, 1, "_kcd"),     // 9: 2 workgroups per CU
    // 10: 8 waves, 2 per SIMD; its whole-tile K-ordered builds lower the wave
    // priority over each K tile (PR 1): 0.3-0.7% faster in ten paired runs
    // (1024 x 8192 x 8192 145.0 against 144.0 TFLOP/s, 2816^3 135.4 against
    // 134.8).
    {"mfma_128x256x32_w64x64_w8_kcd", SGEMM_PATH_MFMA, 128, 256, 32, 512,
     sgk::sgemm_mfma_kc<128, 256, 32, 64, 64, 4, 2, false, 2, 1, 1, 2, false, 1, 0>,
     sgk::sgemm_mfma<128, 256, 32, 64, 64, 4, 0, 1, 2, true, 1, 2, 0, false, true>,
     sgk::sgemm_mfma<128, 256, 32, 64, 64, 4, 0, 1, 2, false, 1, 2, 0, false, true>,
     sgk::sgemm_mfma_kc<128, 256, 32, 64, 64, 4, 2, true, 2, 0, 1, 2, false, 1>, 1, 1, 0,
     sgk::sgemm_mfma_kc<128, 256, 32, 64, 64, 4, 2, false, 2, 1, 1, 2, true, 1, 0>,
     sgk::sgemm_mfma_kc<128, 256, 32, 64, 64, 4, 2, true, 2, 0, 1, 2, true, 1>},
    MFMA_CFG_KCD(64, 64, 32, 32, 32, 4, 4, false, 1, 2, 0, "_kcd"),       // 11: 4 workgroups per CU
    // 12: 8 waves, 2 per SIMD.  Its whole-tile K-ordered builds lower the wave
    // priority over each K tile (PR 1, as 15 does): 0.15-0.6% faster in ten
    // paired runs (2048^3 136.4 against 135.6 TFLOP/s, 2048^2 x 4096 138.7
    // against 138.1); on 14, two workgroups per CU, the same was up to 18%
    // slower (4096 x 3072 x 4096 116.3 against 142.5).
    {"mfma_128x128x64_w32x64_w8_kcd", SGEMM_PATH_MFMA, 128, 128, 64, 512,
     sgk::sgemm_mfma_kc<128, 128, 64, 32, 64, 4, 2, false, 2, 1, 1, 2, false, 1, 0>,
     sgk::sgemm_mfma<128, 128, 64, 32, 64, 4, 0, 1, 2, true, 1, 2, 0, false, true>,
     sgk::sgemm_mfma<128, 128, 64, 32, 64, 4, 0, 1, 2, false, 1, 2, 0, false, true>,
     sgk::sgemm_mfma_kc<128, 128, 64, 32, 64, 4, 2, true, 2, 0, 1, 2, false, 1>, 1, 1, 0,
     sgk::sgemm_mfma_kc<128, 128, 64, 32, 64, 4, 2, false, 2, 1, 1, 2, true, 1, 0>,
     sgk::sgemm_mfma_kc<128, 128, 64, 32, 64, 4, 2, true, 2, 0, 1, 2, true, 1>},
    // 13: the block for at most one tile per CU.  Its 128-bit build (and
    // the one for rows at 4-byte alignment) is two
    // wave groups (KG 2) of two 64 x 32 waves, each group half of every K
    // tile: two MFMAs per k-step and wave instead of one, and per MFMA half
    // the LDS fragment reads of four 32 x 32 waves.  Its 32-bit and checked
    // builds are the register-staged 64 x 64 x 64 block, its split-K and
    // stream-K builds the K-ordered one with four 32 x 32 waves.
    {"mfma_64x64x64_w64x32_kg2_kcd", SGEMM_PATH_MFMA, 64, 64, 64, 256,
     sgk::sgemm_mfma_kc<64, 64, 64, 64, 32, 4, 1, false, 2, 0, 2, 2, false, 1>,
     sgk::sgemm_mfma<64, 64, 64, 32, 32, 4, 0, 1, 2, true, 1, 2, 0, false, true>,
     sgk::sgemm_mfma<64, 64, 64, 32, 32, 4, 0, 1, 2, false, 1, 2, 0, false, true>,
     sgk::sgemm_mfma_kc<64, 64, 64, 32, 32, 4, 2, true, 1, 0, 1, 2, false, 2>, 1, 1, 0,
     sgk::sgemm_mfma_kc<64, 64, 64, 64, 32, 4, 1, false, 2, 0, 2, 2, true, 1>,
     sgk::sgemm_mfma_kc<64, 64, 64, 32, 32, 4, 2, true, 1, 0, 1, 2, true, 2>},
    MFMA_CFG_KCD(128, 128, 32, 64, 32, 4, 4, false, 2, 1, 0, "_w8_kcd"),  // 14: 8 waves, 2 workgroups per CU
    // 15: 7 with 16 waves of 64 x 64, four per SIMD, whole tiles only: its
    // split builds would spill (55-96 registers at the 128-register cap), so
    // split-K and stream-K stay with 7.  Wave priority falls over each K tile
    // (PR 1).  Holding the last k-step over the barrier (DF) measured level
    // here (148.2 against 148.1 TFLOP/s at 8192^3): four waves per SIMD
    // already keep the matrix unit busy across it, so it is not built in.
    {"mfma_256x256x32_w64x64_w16_kcd", SGEMM_PATH_MFMA, 256, 256, 32, 1024,
     sgk::sgemm_mfma_kc<256, 256, 32, 64, 64, 4, 4, false, 2, 1>,
     sgk::sgemm_mfma<256, 256, 32, 64, 64, 4, 0, 1, 4, true, 1, 2, 0, false, true>,
     sgk::sgemm_mfma<256, 256, 32, 64, 64, 4, 0, 1, 4, false, 1, 2, 0, false, true>,
     nullptr, 1, 0, 0,
     sgk::sgemm_mfma_kc<256, 256, 32, 64, 64, 4, 4, false, 2, 1, 1, 2, true>},
    // 16: 15 with K tiles of 16 in a ring of four LDS stages, each tile's
    // loads issued three tiles ahead (sgemm_mfma_kc, STG): a measured
    // alternative to the two-stage double buffer, 3% slower at 4096^3 and
    // 8192^3 (twice the barriers per FLOP), so not chosen.  Its 32-bit and
    // checked builds are the register-staged block of the same tile.
    {"mfma_256x256x16_w64x64_w16_s4_kcd", SGEMM_PATH_MFMA, 256, 256, 16, 1024,
     sgk::sgemm_mfma_kc<256, 256, 16, 64, 64, 4, 4, false, 2, 1, 1, 4>,
     sgk::sgemm_mfma<256, 256, 16, 64, 64, 4, 0, 1, 4, true, 1, 2, 0, false, true>,
     sgk::sgemm_mfma<256, 256, 16, 64, 64, 4, 0, 1, 4, false, 1, 2, 0, false, true>,
     nullptr, 1, 0},
    // 17, 18: small tiles for shapes that cannot give every CU a 64 x 64
    // tile, each tile split over wave groups (KG) so that a workgroup still
    // has four waves: 32 x 32 in four groups of one wave, 32 x 64 in two
    // groups of two.  More, smaller workgroups per CU hide each other's
    // prologue and epilogue (512^3: 47 against 22 TFLOP/s on 64 x 64).
    // Their 32-bit and checked builds are the same block loading 4 bytes
    // per lane straight into LDS, which is slow (the choice takes these
    // blocks only for operands that allow 16-byte loads of A and B); no
    // split builds.
    // RO: the 32 x 64 block reads its A group, B fragments and next A group
    // before the first MFMA (0: 1024^3 105.4 against 104.4 TFLOP/s with 1,
    // ragged 92.3 against 91.6, 1024 x 1024 x 4096 120.6 against 118.4);
    // the 32 x 32 block is level between the orders and keeps 1.
    MFMA_CFG_KG(32, 32, 64, 4, 1, "_kg4_kcd"),
    MFMA_CFG_KG(32, 64, 64, 2, 0, "_kg2_kcd"),
    // 19: 17 with its K tiles in a ring of three LDS stages, each tile's
    // loads issued two tiles ahead (128-bit build; its other builds are
    // 17's): for half a 32 x 32 tile to one per CU and long K, where a lone
    // workgroup per CU otherwise waits for each tile's loads in turn
    // (512 x 512 x 2048 69.7 against 53.9 TFLOP/s, 384 x 384 x 2048 39.3
    // against 30.7, 480 x 480 x 2048 60.9 against 46.4, 512 x 512 x 8192
    // 80.5 against 60.5).  Slower with more tiles per CU (768 x 768 x 4096
    // 80.5 against 87.2), with K up to 1024 (512 x 512 x 1024 61.2 against
    // 64.8), and mixed with fewer tiles (256 x 256 x 2048 17.7 against
    // 20.0, x 4096 19.2 against 15.0; 128 x 512 x 4096 19.3 against 21.9).
    {"mfma_32x32x64_w32x32_kg4_s3_kcd", SGEMM_PATH_MFMA, 32, 32, 64, 256,
     sgk::sgemm_mfma_kc<32, 32, 64, 32, 32, 4, 4, false, 1, 0, 4, 3, false, 1>,
     sgk::sgemm_mfma_kc<32, 32, 64, 32, 32, 1, 4, false, 1, 0, 4, 2, false, 1>,
     sgk::sgemm_mfma_kc<32, 32, 64, 32, 32, 1, 4, false, 1, 0, 4, 2, false, 1>, nullptr, 1, 0, 1,
     sgk::sgemm_mfma_kc<32, 32, 64, 32, 32, 4, 4, false, 1, 0, 4, 2, true, 1>, nullptr},
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

constexpr int kValuDefault = 0;  // 128 x 128 x 16, 8 x 8 per lane, four workgroups per CU
constexpr int kValuWide = 1;     // 128 x 256 x 16, 8 x 16 per lane, two workgroups per CU
// the blocks with A in K order, loaded straight into LDS
constexpr int kKcHuge = 7;       // 256 x 256 x 32, 8 waves, one workgroup per CU
constexpr int kKcLarge4 = 8;     // 128 x 128 x 16, four workgroups per CU
constexpr int kKcShortK = 9;     // 128 x 256 x 16, two workgroups per CU
constexpr int kKcWide = 10;      // 128 x 256 x 32, 8 waves, one workgroup per CU
constexpr int kKcSmall4 = 11;    // 64 x 64 x 32, four workgroups per CU
constexpr int kKcDeep8 = 12;     // 128 x 128 x 64, 8 waves, one workgroup per CU
constexpr int kKcSmall64 = 13;   // 64 x 64 x 64, one tile per CU (two wave groups)
constexpr int kKcMid8 = 14;      // 128 x 128 x 32, 8 waves, two workgroups per CU
constexpr int kKcHuge16 = 15;    // 256 x 256 x 32, 16 waves, one workgroup per CU, whole tiles only
constexpr int kKcTiny4 = 17;     // 32 x 32 x 64 in four wave groups
constexpr int kKcTiny2 = 18;     // 32 x 64 x 64 in two wave groups
constexpr int kKcTiny4Ring = 19; // 17 with three LDS stages
constexpr int kRingMinK = 2048;  // the shortest K at which 19 beats 17

// The machine shape the choices depend on: compute units (tile quantisation,
// stream-K workers, the split-K thresholds and the cut into pieces) and XCDs (the
// workgroup -> tile order).  The choice of tile is a pure function of the
// sizes and this shape, so it is the same on every call and testable without
// a GPU (sgemm_plan_for).
struct Machine {
    long long cus;
    int xcds;
};
constexpr Machine kMI355X = {256, 8};
constexpr int kMaxSplits = 64;
constexpr int kMaxWorkers = 4096;
constexpr int kMaxDevices = 64;

// The current device's shape, read once per device from its attributes
// (MI355X's 256 CUs in 8 XCDs when there is no device to ask, so that the
// host-only queries still answer on a machine without a GPU).
Machine device_machine() {
    static std::once_flag once[kMaxDevices];
    static Machine shape[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return kMI355X;
    }
    std::call_once(once[dev], [dev]() {
        Machine m = kMI355X;
        int cus = 0, xcds = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            cus > 0)
            m.cus = cus;
        // the workgroup -> tile order takes a power of two (8 on an MI355X,
        // 4, 2 or 1 on its partitions); any other count gets the row-major
        // order of one XCD
        if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) == hipSuccess && xcds > 0 &&
            (xcds & (xcds - 1)) == 0)
            m.xcds = xcds;
        else
            m.xcds = 1;
        (void)hipGetLastError();
        shape[dev] = m;
    });
    return shape[dev];
}

// The scratch of sgemm_ws_noalloc: the split-K / stream-K partial tiles of
// one call, in a file-scope device array (one per GPU, held until the
// process ends) instead of a caller's workspace.  Its address comes from
// hipGetSymbolAddress, once per device with that device current: in host
// code the array's name is only a host-side stand-in.
constexpr size_t kScratchBytes = SGEMM_NOALLOC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) float scratch[kScratchBytes / sizeof(float)];

struct ScratchPtr {
    void *ptr;
    int err;  // hipError_t of the lookup
};

ScratchPtr scratch_for_device() {
    static std::once_flag once[kMaxDevices];
    static ScratchPtr cache[kMaxDevices];
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return {nullptr, e != hipSuccess ? (int)e : (int)hipErrorInvalidDevice};
    }
    std::call_once(once[dev], [dev]() {
        void *p = nullptr;
        const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) (void)hipGetLastError();
        cache[dev] = {err == hipSuccess ? p : nullptr, (int)err};
    });
    return cache[dev];
}

// log2 of a power of two
int log2_of(int x) {
    int s = 0;
    while ((1 << (s + 1)) <= x) ++s;
    return s;
}

long long tiles(int M, int N, int bm, int bn) {
    return (long long)((M + bm - 1) / bm) * (long long)((N + bn - 1) / bn);
}

// Fraction of the last round of tiles that keeps the compute units busy:
// t tiles over c CUs take ceil(t / c) rounds of per-CU work.
double quantization(long long t, long long c) {
    const long long rounds = (t + c - 1) / c;
    return rounds == 0 ? 0.0 : (double)t / (double)(rounds * c);
}

// Fraction of the tiles' area that lies inside C: padded rows and columns of
// edge tiles still issue every MFMA.
double fill(int M, int N, int bm, int bn) {
    const long long t = tiles(M, N, bm, bn);
    return t == 0 ? 0.0 : (double)M * (double)N / ((double)t * bm * bn);
}

// Measured on MI355X over every variant with `python -m fp32_gemm_03_amd.tune`
// (cubes 256..10240, 16384^2 x K for K = 128..1024, 1024 x 8192 x 8192,
// 16384 x 1024 x 1024 both ways, 1000 x 1023 x 999, and split-K shapes):
//   * blocks with A in K order, loaded straight into LDS, match or beat the
//     same blocks on the interleaved schedule with A transposed (by 2-3% at
//     128 x 128 x 16, up to 10% on 64 x 64 blocks).  On the 128 x 128 x 32
//     and 128 x 128 x 64 blocks that holds with 8 waves (two per SIMD):
//     with 4 waves of 64 x 64 the K-ordered blocks were 0.5-1% slower than
//     the interleaved ones, with 8 waves 1.5-3% faster (128 x 128 x 32:
//     143.1 against 139.4 TFLOP/s at 4096^3, 143.9 against 140.2 at 6144^3);
//   * a block shape reaches its full-chip rate only once there is a tile for
//     every workgroup slot on the chip (slots = workgroups per CU x 256);
//     below that its workgroups run alone on their CUs and latency shows.
//     Among the shapes that qualify, what decides is the full-chip rate times
//     the share of CUs the last round of tiles keeps busy.  Rates, TFLOP/s:
//     256 x 256 x 32 with 16 waves (1 per CU) 147 (0.25-0.6% above 8 waves
//     on whole rounds; no stream-K build), with 8 waves 146.5,
//     128 x 128 x 16 (4 per CU) 144 (141-145.5 from 6144^3 to 14848^3),
//     128 x 256 x 16 (2 per CU) 144, 128 x 256 x 32 with 8 waves (1 per CU)
//     143, 128 x 128 x 32 with 8 waves (2 per CU) 142.5, 128 x 128 x 64 with
//     8 waves (1 per CU) 139.5, 64 x 64 x 32 (4 per CU) 134 (its rate at
//     2048^3-6144^3; it falls to 117-130 from 8192^3 up, where better-filled
//     blocks win).  With K short the epilogue is a larger
//     share of a tile's time and blocks with more workgroups per CU, which
//     hide one workgroup's epilogue under another's K loop, win: the
//     one-per-CU blocks need K >= 512 and the 128 x 128 ones K >= 256 (at
//     16384^2 x 128 the 128 x 256 x 16 block runs 112 TFLOP/s against 105
//     and 90).  So 8192^3, 4096^3 and 16384 x 1024 x 1024 (whole rounds of
//     256 x 256 blocks) take 256 x 256; 6144^3 to 10240^3 take
//     128 x 128 x 16; 1024 x 8192 x 8192 (one 128 x 256 block per CU) takes
//     128 x 256 x 32; 2048^3 (one 128 x 128 block per CU) 128 x 128 x 64;
//     3072^3 and 5120^3 take 64 x 64 x 32 (5120^3: 135 against 128.5 for
//     128 x 128 x 16); the low-K square takes 128 x 256 x 16;
//   * below that the problem cannot fill the chip: 64 x 64 blocks, split
//     along K when K is long (select_splits).  With at most one tile per CU
//     the K-ordered 64 x 64 x 64 block, which halves the barriers per FLOP,
//     is 5-8% faster than 64 x 64 x 32 (1024^3 96.5 against 91.4 TFLOP/s,
//     1000 x 1023 x 999 77 against 71, 1024 x 1024 x 4096 109 against
//     102); with more tiles, 64 x 64 x 32 at four workgroups per CU is
//     (3072^3 121 against 116, 5120^3 131 against 125).
// Stream-K (with a workspace): a block whose tiles do not divide evenly over
// the CUs runs the whole rounds as usual and spreads the K tiles of the rest
// over one worker per CU, so every CU ends at about the same time.  One per
// CU also for the blocks that run two or four workgroups per CU: measured
// 3-5% faster than one per workgroup slot at 3072^3 and 2560^2 x 4096 on
// 128 x 128 x 32, and up to 1% at 5120^3-7168^3 on 128 x 128 x 16.  Scored
// as the block's full-chip rate times kStreamKShare, the measured cost of the
// partial tiles and their summing pass, when each worker gets at least
// kStreamKMinK K tiles, and priced by kTileStartK below.  So with a
// workspace the large squares whose 256 x 256 tiles leave a partial round run
// stream-K on 256 x 256 x 32 at 141-146 TFLOP/s, 3-5% above the best
// whole-tile block (5120^3, 7168^3, 13824^3); where stream-K's gain was 1% or
// less, the price leaves whole tiles (6144^3 0.4% faster on 128 x 128 x 16,
// 10240^3 and 12800^3 about 1% slower).
constexpr double kStreamKShare = 0.985;
constexpr int kStreamKMinK = 8;
// A fixed cost per tile (its first loads, its write-back of C), as this many
// more steps of K, where nothing overlaps it: on the stream-K workers'
// partial tiles, and on the 256 x 256 tiles of a cut's first piece (one
// workgroup per CU).  For stream-K, over 57 shapes 1024-8192 wide where the
// price changed the plan of sgemm_ws, the new plans ran 3.5% faster in
// geometric mean: 5.1% with K = 1024 (33 shapes; 3584 x 8192 x 1024 on
// whole 128 x 128 x 16 tiles 142.9 against 130.9 stream-K on 256 x 256), 2.3%
// with K = 2048, level at 4096; five ran 1-4% slower (7680 x 6656 x 1024,
// 4096 x 5120 x 4096).  Smaller prices took fewer of the gains (25: 1.6%, 50:
// 2.4%).
constexpr double kTileStartK = 75.0;
// K from which stream-K on 64 x 64 x 32 beats the 64 x 64 x 64 block at one
// or two tiles per CU (1280^2 x 4096 yes, 1280^3 and 1408^3 no)
constexpr int kStreamKLongK = 2048;

// Candidate rates, TFLOP/s, of the two 256 x 256 x 32 blocks and of 64 x 64
// blocks that cannot fill the chip (256 rows of 7168^2 x 7168 ran 114 on
// 64 x 64 x 32; 1024^3 runs 96 on 64 x 64 x 64).
constexpr double kHuge16Rate = 147.0;
constexpr double kSmallRate = 110.0;
// The 64 x 64 x 32 block (four per CU) against the 32 x 64 wave-group block
// (three per CU) where both have several tiles per CU: the same balance of
// tiles over the CUs favours the former by 3.5% (3072^3 133.9 against
// 129.2, 4608^3 130.9 against 126.7), but the finer 32 x 64 grid often
// balances better (1536^3 110.7 against 96.8 TFLOP/s, 2304^3 118.5 against
// 112.6, 3072 x 1536 x 2048 125.3 against 117.6).
// Below K = 1024 the 32 x 64 block's fixed costs per tile lose (3584^2 x 512
// 112.5 against 121.5, 2560^2 x 256 94.8 against 105.4, K = 128: 16-20%
// slower), so it is weighed only from there.
constexpr double kSmall4Rate = 134.0;
constexpr double kTiny2Rate = 129.3;
constexpr int kTiny2MinK = 1024;
// A block of one workgroup per CU also qualifies with its tiles just short of
// one round, at least this share of the CUs busy (scored by that share):
// over 49 shapes 1024-7680 wide where that changed the choice (to 128 x 256
// from 128 x 128, or to 256 x 256 from 128 x 256), every one ran as fast or
// faster, 2.6% in geometric mean (2816^3 135.2 against 131.1, 3584 x 4608 x
// 4096 145.5 against 141.8).  From 70% of the CUs the smaller blocks' finer
// grids won back (1536 x 2048 x 2048 on 128 x 128 tiles: 102.4 against 129.2
// on 64 x 64).
constexpr double kShortRoundShare = 0.9;

// The variant for a whole-tile (or, with streamk, stream-K) launch on a
// machine of m.cus compute units; *score gets its predicted TFLOP/s (rate x
// the busy share of the last round x the share of the tiles' area inside C).
// small_ok: the operands allow the small blocks' 16-byte loads (rows of A and
// B 4-byte aligned, in-tile offsets within 31 bits), which they need to be
// fast (their other builds load 4 bytes per lane into LDS).
int choose(const Machine &m, int path, int M, int N, int K, bool streamk, bool small_ok, int *workers,
           double *score_out = nullptr) {
    if (workers) *workers = 0;
    if (score_out) *score_out = 0.0;
    if (M < 0) return -1;
    if (N < 0) return -2;
    if (K < 0) return -3;
    const long long cus = m.cus;
    if (path == SGEMM_PATH_VALU) {
        // The 8 x 16 micro-tile reads 25% less LDS per FMA and is 11-19%
        // faster at 4096^3 and 8192^3, but only where its 128 x 256 blocks
        // fill whole rounds of the CUs and K is long: at 5120^3 to 10240^3,
        // at 16384^2 x 128 and with fewer blocks than slots the 8 x 8 tile
        // is as fast or faster (measured over the same shapes as below).
        const long long t = tiles(M, N, 128, 256);
        if (t >= 2 * cus && t % cus == 0 && K >= 1024) return kValuWide;
        return kValuDefault;
    }
    if (path != SGEMM_PATH_AUTO && path != SGEMM_PATH_MFMA) return SGEMM_ERR_PATH;
    struct Candidate {
        int variant;
        double rate;         // full-chip TFLOP/s, measured
        int per_cu;          // workgroups resident per CU
        int min_k;           // shortest K at which that rate holds
    };
    static const Candidate cand[] = {{kKcHuge16, kHuge16Rate, 1, 512}, {kKcHuge, 146.5, 1, 512},
                                     {kKcLarge4, 144.0, 4, 256},
                                     {kKcShortK, 144.0, 2, 0},  {kKcWide, 143.0, 1, 512},
                                     {kKcMid8, 142.5, 2, 256},  {kKcDeep8, 139.5, 1, 1024},
                                     {kKcSmall4, kSmall4Rate, 4, 0}};
    int best = -1, best_workers = 0;
    double best_score = -1.0;
    for (const Candidate &c : cand) {
        const Variant &v = kVariants[c.variant];
        const long long t = tiles(M, N, v.bm, v.bn);
        const long long slots = c.per_cu * cus;
        const bool short_round = c.per_cu == 1 && t < slots;
        if ((short_round ? (double)t < kShortRoundShare * (double)slots : t < slots) || K < c.min_k) continue;
        const double f = fill(M, N, v.bm, v.bn);
        double score = c.rate * quantization(t, cus) * f;
        int w = 0;
        const long long rest = t % cus, kt = (K + v.bk - 1) / v.bk;
        const double sk_score = c.rate * kStreamKShare * f * K / (K + kTileStartK);
        if (streamk && v.streamk && !short_round && rest > 0 && rest * kt >= kStreamKMinK * cus &&
            sk_score > score) {
            score = sk_score;
            w = (int)cus;
        }
        if (score > best_score) {
            best_score = score;
            best = c.variant;
            best_workers = w;
        }
    }
    // the 32 x 64 block where its tiles balance better over the CUs
    auto tiny2_score = [&]() {
        if (K < kTiny2MinK) return 0.0;
        return kTiny2Rate * quantization(tiles(M, N, 32, 64), cus) * fill(M, N, 32, 64);
    };
    if (best == kKcSmall4 && best_workers == 0 && small_ok && tiny2_score() > best_score) {
        best = kKcTiny2;
        best_score = tiny2_score();
    }
    if (best < 0) {
        // No block fills the chip (measured over cubes 256-1920 and
        // rectangles; TFLOP/s).  With operands that allow 16-byte loads
        // (128-bit ones here; rows at 4-byte alignment run within 1-5%):
        //   * at most three 32 x 32 tiles per CU: the 32 x 32 block in four
        //     wave groups (256^3 6.6 against 4.5 on 64 x 64, 512^3 47 against
        //     22, 768^3 69 against 54, 512 x 512 x 8192 62 against 29);
        //   * at most three 32 x 64 tiles per CU (three of its workgroups fit
        //     a CU's LDS, so that is one round): the 32 x 64 block in two
        //     wave groups (1024^3 104 against 99, 1024 x 1024 x 4096 120
        //     against 113, 1152^3 100 against 73, 1536 x 1024 x 2048 122
        //     against 92, 3072 x 512 x 1024 113 against 86);
        //   * at most two 64 x 64 tiles per CU (one round of two per CU): the
        //     64 x 64 x 64 block (1408^3 116 against 110, 2048 x 1024 x 2048
        //     127 against 120), unless stream-K on 64 x 64 x 32 shares long K
        //     ranges (1280^2 x 4096: 110 against 102).
        // Other operands take the 64 x 64 x 64 block up to two tiles per CU
        // as well (32-bit builds: 1151^3 69 against 67, 2047 x 1023 x 1023
        // 106 against 100).
        // Otherwise the 64 x 64 x 32 block at four per CU; with more tiles than CUs but
        // not a whole number per CU, stream-K over one worker per CU evens
        // out the K tiles each CU runs (1536^3: 110 against 96).  With at
        // most one 64 x 64 tile per CU, the deeper K tile, and select_splits
        // may split K.
        const Variant &v = kVariants[kKcSmall4];
        const long long t = tiles(M, N, v.bm, v.bn), rest = t % cus;
        const long long kt = (K + v.bk - 1) / v.bk;
        const bool sk = streamk && rest > 0 && rest * kt >= kStreamKMinK * cus;
        if (small_ok && tiles(M, N, 32, 32) <= 3 * cus) {
            if (score_out) *score_out = kSmallRate * fill(M, N, 32, 32);
            // between half a tile and one tile per CU and long K: the
            // three-stage ring
            const long long t32 = tiles(M, N, 32, 32);
            return t32 <= cus && 2 * t32 >= cus && K >= kRingMinK ? kKcTiny4Ring : kKcTiny4;
        }
        if (small_ok && tiles(M, N, 32, 64) <= 3 * cus) {
            if (score_out) *score_out = kSmallRate * fill(M, N, 32, 64);
            return kKcTiny2;
        }
        if (score_out) *score_out = kSmallRate * fill(M, N, v.bm, v.bn);
        if (t <= cus || (t <= 2 * cus && !(sk && K >= kStreamKLongK))) return kKcSmall64;
        if (sk && workers) {
            *workers = (int)cus;
            return kKcSmall4;
        }
        const double s4 = kSmall4Rate * quantization(t, cus) * fill(M, N, v.bm, v.bn);
        if (small_ok && tiny2_score() > s4) {
            if (score_out) *score_out = tiny2_score();
            return kKcTiny2;
        }
        // more than two tiles per CU: the block's own rate holds
        if (score_out) *score_out = s4;
        return kKcSmall4;
    }
    if (workers) *workers = best_workers;
    if (score_out) *score_out = best_score;
    return best;
}

int select_variant(const Machine &m, int path, int M, int N, int K, bool small_ok) {
    return choose(m, path, M, N, K, false, small_ok, nullptr);
}

// The first piece's 256 x 256 tiles run one workgroup per CU: each pays its
// first loads and its write-back of C with nothing to overlap them, priced
// as kTileStartK more steps of K per tile.  Over 93 shapes measured both
// ways (cubes 4352-11776, rectangles 2048 to 20000 wide, K 512-8192),
// pricing the rate alone with K of 2048 or more took 75 cuts, 12 of them up
// to 3% slower than one launch; with this price the model takes 51, of which
// 49 ran 0.2-9.3% faster and two 2.4% and 3.1% slower (3.6% faster in
// geometric mean).  With K of 512, 8 of 10 cuts predicted 2% faster ran
// slower.
constexpr int kPiecesMinK = 1024;

struct Pieces {
    int rows = 0, cols = 0;  // the first piece; rows == 0: one launch
    int variant = -1;        // the first piece's block
};

// The blocks a cut's first piece may run on, one workgroup per CU each: the
// 256 x 256 block first; the others only where it gives no cut, and only
// with K of at least kPiecesOtherMinK.  Measured over 36 shapes 2048-6144
// wide where only the others gave a cut: 1.8% faster than one launch in
// geometric mean (5376 x 3328 x 3072 on 128 x 256 tiles 137.9 against 129.9,
// 4608 x 3072 x 4096 on 128 x 128 140.4 against 132.8), 3 of the 4 slower
// ones (1.0-1.6%) with K = 1024.
struct FirstPiece {
    int variant, bm, bn;
    double rate;
};
constexpr int kPiecesOtherMinK = 1536;

// Without a workspace there is no stream-K, and a partial last round of
// tiles leaves CUs idle.  C can instead be cut into pieces, one launch each:
// a first piece of rows x cols whose tiles fill their rounds (at least 96% of
// the last one busy) on a block of one workgroup per CU (FirstPiece), the
// columns right of it over those rows, and the rows below it over every
// column, each of the two with the block chosen for it.  cols == N cuts by
// rows alone (the first piece then pads its last tile column), rows == M by
// columns alone.  Returns rows = 0 when one launch is predicted within 2% of
// the best cut.  Measured against one launch, in the same process: 4352^3
// 141.0 against 128.9 TFLOP/s, 5120^3 142.8 against 137.4, 7168^3 144.7
// against 138.0, 11264^3 146.1 against 141.6; at 5120^3, 7168^3, 9216^3,
// 11264^3 and 13824^3 the cut the model picked (without the price of a
// tile's start) ran within 0.3% of the best of up to 40 cuts tried.  Only the
// last 64 block rows and 32 block columns are tried as the first piece's
// edges.
Pieces split_pieces(const Machine &m, int M, int N, int K, bool small_ok) {
    Pieces best;
    if (K < kPiecesMinK || M < 512) return best;
    double single = 0.0;
    if (choose(m, SGEMM_PATH_AUTO, M, N, K, false, small_ok, nullptr, &single) < 0 || single <= 0.0) return best;
    const double per_elem = 2.0 * (double)K;
    const double t_single = per_elem * M * (double)N / single;
    // No block's predicted rate exceeds the 256 x 256 block's, so no cut can
    // beat a launch predicted within 2% of it (8192^3, whole rounds), and a
    // cut whose first piece alone, with the rest at that rate, is slower
    // than the best so far need not be priced further.
    if (single >= 0.98 * kHuge16Rate) return best;
    double best_t = 0.98 * t_single;
    // predicted time of an m1 x n1 piece with the block chosen for it
    auto piece = [&](int m1, int n1) {
        if (m1 == 0 || n1 == 0) return 0.0;
        double s = 0.0;
        if (choose(m, SGEMM_PATH_AUTO, m1, n1, K, false, small_ok, nullptr, &s) < 0 || s <= 0.0) return -1.0;
        return per_elem * m1 * (double)n1 / s;
    };
    static const FirstPiece firsts[] = {{kKcHuge16, 256, 256, kHuge16Rate},
                                        {kKcWide, 128, 256, 143.0},
                                        {kKcDeep8, 128, 128, 139.5}};
    for (const FirstPiece &fp : firsts) {
        // the other blocks only where the 256 x 256 one gives no cut
        if (fp.variant != kKcHuge16 && (best.variant == kKcHuge16 || K < kPiecesOtherMinK)) break;
        const long long nbn = (N + fp.bn - 1) / fp.bn;
        const long long rb_hi = M / fp.bm, rb_lo = rb_hi > 64 ? rb_hi - 64 : 1;
        const long long cb_hi = (N - 1) / fp.bn, cb_lo = cb_hi > 32 ? cb_hi - 32 : 1;
        for (long long rb = rb_hi; rb >= rb_lo; --rb) {
            const int m1 = (int)(rb * fp.bm);
            double t_below = -2.0;  // the piece below, chosen once per rb
            // cb = nbn: every column, padded (a cut by rows only)
            for (long long cb = nbn; cb >= cb_lo; --cb) {
                const bool full = cb == nbn;
                if (full && m1 == M) continue;  // that is one launch
                const long long t = rb * cb;
                if (t < m.cus) break;
                const double q = quantization(t, m.cus);
                if (q < 0.96) continue;
                const int n1 = full ? N : (int)(cb * fp.bn);
                const double fill = full ? (double)N / (double)(nbn * fp.bn) : 1.0;
                const double t_first = per_elem * m1 * (double)n1 / (fp.rate * q * fill) * (K + kTileStartK) / K;
                const double rest = per_elem * ((double)M * N - (double)m1 * n1) / kHuge16Rate;
                if (t_first + rest >= best_t) continue;
                if (t_below == -2.0) t_below = piece(M - m1, N);
                if (t_below < 0.0) break;
                const double t_right = full ? 0.0 : piece(m1, N - n1);
                if (t_right < 0.0) continue;
                const double t_split = t_first + t_right + t_below;
                if (t_split < best_t) {
                    best_t = t_split;
                    best.rows = m1;
                    best.cols = n1;
                    best.variant = fp.variant;
                }
            }
        }
    }
    return best;
}

// Split count for a variant when a workspace is available (measured on
// MI355X: 512 x 512 x 8192 runs 3.5x faster in 8 parts, 768^3 13% faster in
// 3, 1024 x 1024 x 4096 about 10% faster in 2, while 1024^3 loses): split
// only when the tiles alone leave CUs idle, into enough parts for about two
// workgroups per CU, keeping at least 256 of K per part (1024 when there is
// already a tile for every CU) so the per-workgroup prologue and the extra
// pass over the partials stay small.  Only the latency block splits: the
// blocks chosen by rate have a tile for every one of their workgroup slots
// on the chip already.
int select_splits(const Machine &m, int variant, int M, int N, int K) {
    if (M <= 0 || N <= 0 || K <= 0 || (variant != kKcSmall4 && variant != kKcSmall64)) return 1;
    const Variant &v = kVariants[variant];
    if (v.split4 == nullptr) return 1;
    const long long t = tiles(M, N, v.bm, v.bn);
    if (t > m.cus) return 1;
    long long s = 2 * m.cus / t;
    const long long k_min = t < m.cus ? 256 : 1024;
    if (s > K / k_min) s = K / k_min;
    if (s > kMaxSplits) s = kMaxSplits;
    return s < 2 ? 1 : (int)s;
}

// With a workspace, a shape the small blocks would take runs split-K on the
// 64 x 64 x 64 block instead when K is long enough for 4 parts or more
// (512 x 512 x 8192 in 8 parts: 99.6 TFLOP/s against 62 on 32 x 32; with 2
// or 3 parts the small blocks win: 512^3 47 against 26, 768^3 69 against
// 57, 1024 x 1024 x 4096 120 against 115).  Against the three-stage ring
// with a 32 x 32 tile for every CU, parts need at least 512 of K (512 x 512
// x 2048 in 8 parts: 60.9 against 69.7 for the ring; x 4096: 81.5 against
// 76.4); with fewer tiles than half the CUs the split always wins (256 x 256
// x 4096: 42.7 against 19.2).  A split into no more workgroups than the
// small block has loses (512 x 512 x 1024 in 4 parts: 49.3 against 64.8;
// 256 x 256 x 1024: 13.1 against 16.8), so it needs more.
constexpr int kTinySplitMin = 4;
constexpr int kRingSplitMinPart = 512;

// What sgemm_ws (with_workspace) or sgemm (without) runs for these sizes:
// the variant, split count, stream-K workers and the first piece of a cut
// into several launches (rows 0: none).  Returns 0 or a negative argument code.
// load16: the operands allow 16-byte loads of A and B (loads16 below),
// which the small blocks, split-K and stream-K need: loading 4 bytes per
// lane straight into LDS, split launches measured slower than one launch of
// whole tiles (767^3 in 3 parts 27.6 against 47.5 TFLOP/s, 1535^3 stream-K
// 60.0 against 88.6, 1023 x 1023 x 4095 in 2 parts 62.7 against 100.2), and
// the small blocks slower than the 64 x 64 one.
int plan(const Machine &m, int M, int N, int K, bool with_workspace, bool load16, int *variant,
         int *splits, int *workers, Pieces *pieces) {
    int w = 0;
    const bool parts = with_workspace && load16;
    int v = choose(m, SGEMM_PATH_AUTO, M, N, K, parts, load16, &w);
    if (v < 0) return v;
    int sp = 1;
    Pieces pc;
    if (parts && w == 0) {
        if (v == kKcTiny4 || v == kKcTiny2 || v == kKcTiny4Ring) {
            const int s = select_splits(m, kKcSmall64, M, N, K);
            const bool ring_wins = v == kKcTiny4Ring && 2 * tiles(M, N, 32, 32) >= m.cus &&
                                   K / (s > 0 ? s : 1) < kRingSplitMinPart;
            // the parts must outnumber the small block's workgroups
            const long long small_wgs = v == kKcTiny2 ? tiles(M, N, 32, 64) : tiles(M, N, 32, 32);
            if (s >= kTinySplitMin && tiles(M, N, 64, 64) * s > small_wgs && !ring_wins) {
                v = kKcSmall64;
                sp = s;
            }
        } else {
            sp = select_splits(m, v, M, N, K);
        }
    }
    if (w == 0 && sp == 1) pc = split_pieces(m, M, N, K, load16);
    if (variant) *variant = v;
    if (splits) *splits = sp;
    if (workers) *workers = w;
    if (pieces) *pieces = pc;
    return SGEMM_OK;
}

int check_args(int M, int N, int K, float alpha, const float *A, int lda,
               const float *B, int ldb, const float *C, int ldc) {
    if (M < 0) return -1;
    if (N < 0) return -2;
    if (K < 0) return -3;
    const bool reads_ab = alpha != 0.0f && K > 0 && M > 0 && N > 0;
    if (reads_ab && A == nullptr) return -5;
    if (lda < (K > 1 ? K : 1)) return -6;
    if (reads_ab && B == nullptr) return -7;
    if (ldb < (N > 1 ? N : 1)) return -8;
    if (M > 0 && N > 0 && C == nullptr) return -10;
    if (ldc < (N > 1 ? N : 1)) return -11;
    return SGEMM_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

// Whether the operands allow 16-byte loads of A and B (the BUFFER_128 or
// BUFFER_128_AB builds): A, B and C 4-byte aligned, and the in-tile byte
// offsets of a 32 x 64 x 64 block below 2^31 (a larger block's launch
// checks its own with buffer_offsets_ok).
bool loads16(const float *A, int lda, const float *B, int ldb, const float *C, int ldc) {
    const long long lim = 1LL << 31;
    const bool offsets = 33LL * lda * 4 < lim && 65LL * ldb * 4 + 64 * 4 < lim && 33LL * ldc * 4 < lim;
    return offsets && aligned4(A) && aligned4(B) && aligned4(C);
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace of a split-K launch: the partial tiles, float [tile][split][bm*bn].
size_t splitk_bytes(const Variant &v, int splits, int M, int N) {
    return round_up((size_t)splits * (size_t)tiles(M, N, v.bm, v.bn) * v.bm * v.bn * 4, 256);
}

// Workspace of a stream-K launch: two partial tiles per worker,
// float [worker][2][bm*bn].
size_t streamk_bytes(const Variant &v, int workers) {
    return round_up((size_t)workers * 2 * v.bm * v.bn * 4, 256);
}

// Buffer accesses form byte offsets inside one block tile in 31 bits.
bool buffer_offsets_ok(const Variant &v, int lda, int ldb, int ldc) {
    const long long lim = 1LL << 31;
    return (long long)(v.bm + 1) * lda * 4 < lim && (long long)(v.bk + 1) * ldb * 4 + (long long)v.bn * 4 < lim &&
           (long long)(v.bm + 1) * ldc * 4 < lim;
}

int launch(const Machine &m, int variant, int access, int splits, int workers, void *workspace,
           size_t workspace_bytes, int M, int N, int K, float alpha, const float *A, int lda,
           const float *B, int ldb, float beta, float *C, int ldc, hipStream_t stream) {
    const int rc = check_args(M, N, K, alpha, A, lda, B, ldb, C, ldc);
    if (rc != SGEMM_OK) return rc;
    if (variant < 0 || variant >= kNumVariants) return SGEMM_ERR_VARIANT;
    if (access < SGEMM_ACCESS_AUTO || access > SGEMM_ACCESS_BUFFER_128_AB) return SGEMM_ERR_ACCESS;
    if (splits < 1 || splits > kMaxSplits) return SGEMM_ERR_SPLITS;
    if (splits > 1 && kVariants[variant].split4 == nullptr) return SGEMM_ERR_SPLITS;
    if (workers < 0 || workers > kMaxWorkers || (workers > 0 && splits > 1)) return SGEMM_ERR_SPLITS;
    if (workers > 0 && (!kVariants[variant].streamk || kVariants[variant].split4 == nullptr))
        return SGEMM_ERR_SPLITS;
    if (M == 0 || N == 0) return SGEMM_OK;
    const bool no_product = alpha == 0.0f || K == 0;
    if (no_product && beta == 1.0f) return SGEMM_OK;

    const Variant &v = kVariants[variant];
    if (no_product) {  // C = beta * C needs no K split
        splits = 1;
        workers = 0;
    }
    const long long ntiles = tiles(M, N, v.bm, v.bn);
    // stream-K: the last ntiles % workers tiles are shared by the workers
    const long long shared = workers > 0 ? ntiles % workers : 0;
    if (shared == 0) workers = 0;  // whole rounds: every tile whole
    const long long grid = workers > 0 ? ntiles - shared + workers : ntiles * splits;
    if (ntiles * splits > INT_MAX || grid > INT_MAX) return SGEMM_ERR_TOO_LARGE;

    Args a;
    a.M = M;
    a.N = N;
    a.K = no_product ? 0 : K;
    a.alpha = alpha;
    a.beta = beta;
    a.A = A;
    a.B = B;
    a.C = C;
    a.lda = lda;
    a.ldb = ldb;
    a.ldc = ldc;
    a.splits = 1;
    a.partial = nullptr;
    a.phase = 0;
    a.sk_whole = 0;
    a.sk_workers = 0;
    a.xcd_shift = log2_of(m.xcds);
    const bool buf_ok = buffer_offsets_ok(v, lda, ldb, ldc);
    // 128-bit accesses to B and C need 16-byte aligned bases and every row
    // start a multiple of 4 floats; N % 4 == 0 keeps each 4-wide piece wholly
    // inside or wholly outside the matrix.  A is read 32 bits at a time, or,
    // by the variants that read it along K, 128 bits at a time under the
    // same rules with K and lda in place of N and ldb.
    const bool vec4 = (N % 4 == 0) && (ldb % 4 == 0) && (ldc % 4 == 0) &&
                      aligned16(B) && aligned16(C) &&
                      (!v.a128 || ((K % 4 == 0) && (lda % 4 == 0) && aligned16(A)));
    // 16-byte loads of A and B need only 4-byte aligned rows: a buffer load
    // of 16 bytes at a 4-byte aligned offset reads them, and its range check
    // is per 4 bytes, so a load that straddles a matrix's end keeps what lies
    // inside (checked on gfx950 with an in-bounds probe)
    const bool vec4u = v.vec4u != nullptr && aligned4(A) && aligned4(B) && aligned4(C);
    KernelFn fn;
    switch (access) {
        case SGEMM_ACCESS_BUFFER_128:
            if (!buf_ok || !vec4) return SGEMM_ERR_ACCESS;
            fn = v.vec4;
            break;
        case SGEMM_ACCESS_BUFFER_32:
            if (!buf_ok) return SGEMM_ERR_ACCESS;
            fn = v.vec1;
            break;
        case SGEMM_ACCESS_CHECKED:
            fn = v.generic;
            break;
        case SGEMM_ACCESS_BUFFER_128_AB:
            if (!buf_ok || !vec4u) return SGEMM_ERR_ACCESS;
            fn = v.vec4u;
            break;
        default:
            fn = !buf_ok ? v.generic : (vec4 ? v.vec4 : (vec4u ? v.vec4u : v.vec1));
            break;
    }
    if (fn == v.generic && v.generic_buf && !buf_ok) return SGEMM_ERR_ACCESS;
    if (splits > 1 || workers > 0) {
        // split-K and stream-K kernels exist for buffer accesses only
        if (fn == v.generic) return SGEMM_ERR_ACCESS;
        const size_t need = workers > 0 ? streamk_bytes(v, workers) : splitk_bytes(v, splits, M, N);
        if (workspace == nullptr || workspace_bytes < need || ((uintptr_t)workspace & 255u) != 0)
            return SGEMM_ERR_WORKSPACE;
        // (only the 16-byte load builds: 4 bytes per lane, a split launch
        // is slower than whole tiles)
        if (fn == v.vec4) fn = v.split4;
        else if (fn == v.vec4u && v.split4u) fn = v.split4u;
        else return SGEMM_ERR_ACCESS;
        a.splits = splits;
        a.partial = static_cast<float *>(workspace);
        if (workers > 0) {
            a.phase = 2;
            a.sk_whole = (int)(ntiles - shared);
            a.sk_workers = workers;
        }
    }

    (void)hipGetLastError();  // drop any stale error so the code below is this launch's
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(v.threads), 0, stream, a);
    hipError_t err = hipGetLastError();
    if (err == hipSuccess && (splits > 1 || workers > 0)) {
        // the summing phase on the same stream: it starts after every
        // partial is written (split-K: one workgroup per tile; stream-K: one
        // per shared tile)
        a.phase = workers > 0 ? 3 : 1;
        const long long grid2 = workers > 0 ? shared : ntiles;
        hipLaunchKernelGGL(fn, dim3((unsigned)grid2), dim3(v.threads), 0, stream, a);
        err = hipGetLastError();
    }
    return err == hipSuccess ? SGEMM_OK : (int)err;
}

// C cut into pieces: rows x cols at the top left on the first piece's block,
// then the columns right of it over the same rows and the rows below it over
// every column, each with the block chosen for it; one launch each, on the
// same stream.  Moving B and C by cols columns keeps their alignment (cols is
// a multiple of 128).
int launch_pieces(const Machine &m, Pieces pc, int M, int N, int K, float alpha, const float *A, int lda,
                  const float *B, int ldb, float beta, float *C, int ldc, hipStream_t stream) {
    int rc = launch(m, pc.variant, SGEMM_ACCESS_AUTO, 1, 0, nullptr, 0, pc.rows, pc.cols, K, alpha, A, lda,
                    B, ldb, beta, C, ldc, stream);
    if (rc != SGEMM_OK) return rc;
    if (pc.cols < N) {
        const int n2 = N - pc.cols;
        const float *B2 = B + pc.cols;
        float *C2 = C + pc.cols;
        const int v2 = select_variant(m, SGEMM_PATH_AUTO, pc.rows, n2, K, loads16(A, lda, B2, ldb, C2, ldc));
        if (v2 < 0) return v2;
        rc = launch(m, v2, SGEMM_ACCESS_AUTO, 1, 0, nullptr, 0, pc.rows, n2, K, alpha, A, lda, B2, ldb, beta,
                    C2, ldc, stream);
        if (rc != SGEMM_OK) return rc;
    }
    if (pc.rows == M) return SGEMM_OK;
    const float *A3 = A + (size_t)pc.rows * lda;
    float *C3 = C + (size_t)pc.rows * ldc;
    const int v3 = select_variant(m, SGEMM_PATH_AUTO, M - pc.rows, N, K, loads16(A3, lda, B, ldb, C3, ldc));
    if (v3 < 0) return v3;
    return launch(m, v3, SGEMM_ACCESS_AUTO, 1, 0, nullptr, 0, M - pc.rows, N, K, alpha, A3, lda, B, ldb, beta,
                  C3, ldc, stream);
}

}  // namespace

extern "C" {

int sgemm(int M, int N, int K, float alpha, const float *A, int lda,
          const float *B, int ldb, float beta, float *C, int ldc,
          hipStream_t stream) {
    return sgemm_path(SGEMM_PATH_AUTO, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int sgemm_path(int path, int M, int N, int K, float alpha, const float *A,
               int lda, const float *B, int ldb, float beta, float *C, int ldc,
               hipStream_t stream) {
    const int rc = check_args(M, N, K, alpha, A, lda, B, ldb, C, ldc);
    if (rc != SGEMM_OK) return rc;
    const Machine m = device_machine();
    const bool small = loads16(A, lda, B, ldb, C, ldc);
    const int v = select_variant(m, path, M, N, K, small);
    if (v < 0) return v;
    if (path != SGEMM_PATH_VALU) {
        const Pieces pc = split_pieces(m, M, N, K, small);
        if (pc.rows > 0) return launch_pieces(m, pc, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
    }
    return launch(m, v, SGEMM_ACCESS_AUTO, 1, 0, nullptr, 0, M, N, K, alpha, A, lda, B, ldb, beta, C,
                  ldc, stream);
}

int sgemm_variant(int variant, int M, int N, int K, float alpha,
                  const float *A, int lda, const float *B, int ldb, float beta,
                  float *C, int ldc, hipStream_t stream) {
    return launch(device_machine(), variant, SGEMM_ACCESS_AUTO, 1, 0, nullptr, 0, M, N, K, alpha, A,
                  lda, B, ldb, beta, C, ldc, stream);
}

int sgemm_variant_access(int variant, int access, int M, int N, int K, float alpha,
                         const float *A, int lda, const float *B, int ldb, float beta,
                         float *C, int ldc, hipStream_t stream) {
    return launch(device_machine(), variant, access, 1, 0, nullptr, 0, M, N, K, alpha, A, lda, B, ldb,
                  beta, C, ldc, stream);
}

int sgemm_splitk(int variant, int splits, int M, int N, int K, float alpha,
                 const float *A, int lda, const float *B, int ldb, float beta,
                 float *C, int ldc, void *workspace, size_t workspace_bytes,
                 hipStream_t stream) {
    return launch(device_machine(), variant, SGEMM_ACCESS_AUTO, splits, 0, workspace, workspace_bytes,
                  M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

size_t sgemm_splitk_workspace_size(int variant, int splits, int M, int N) {
    if (variant < 0 || variant >= kNumVariants || splits < 1 || splits > kMaxSplits || M < 0 ||
        N < 0)
        return 0;
    if (splits == 1 || M == 0 || N == 0 || kVariants[variant].split4 == nullptr) return 0;
    return splitk_bytes(kVariants[variant], splits, M, N);
}

int sgemm_streamk(int variant, int workers, int M, int N, int K, float alpha,
                  const float *A, int lda, const float *B, int ldb, float beta,
                  float *C, int ldc, void *workspace, size_t workspace_bytes,
                  hipStream_t stream) {
    if (workers < 1) return SGEMM_ERR_SPLITS;
    return launch(device_machine(), variant, SGEMM_ACCESS_AUTO, 1, workers, workspace, workspace_bytes,
                  M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

size_t sgemm_streamk_workspace_size(int variant, int workers) {
    if (variant < 0 || variant >= kNumVariants || workers < 1 || workers > kMaxWorkers) return 0;
    if (!kVariants[variant].streamk || kVariants[variant].split4 == nullptr) return 0;
    return streamk_bytes(kVariants[variant], workers);
}

int sgemm_select_splits(int M, int N, int K) {
    int sp = 1;
    const int rc = plan(device_machine(), M, N, K, true, true, nullptr, &sp, nullptr, nullptr);
    return rc < 0 ? rc : sp;
}

int sgemm_ws_plan(int M, int N, int K, int *variant, int *splits, int *workers) {
    return plan(device_machine(), M, N, K, true, true, variant, splits, workers, nullptr);
}

int sgemm_plan_for(int compute_units, int M, int N, int K, int with_workspace, int operands_load16,
                   int *variant, int *splits, int *workers, int *rows) {
    return sgemm_plan_pieces_for(compute_units, M, N, K, with_workspace, operands_load16, variant, splits,
                                 workers, rows, nullptr, nullptr);
}

int sgemm_plan_pieces_for(int compute_units, int M, int N, int K, int with_workspace, int operands_load16,
                          int *variant, int *splits, int *workers, int *rows, int *cols, int *first_variant) {
    if (compute_units < 1 || compute_units > (1 << 20)) return SGEMM_ERR_MACHINE;
    const Machine m = {compute_units, kMI355X.xcds};
    Pieces pc;
    const int rc = plan(m, M, N, K, with_workspace != 0, operands_load16 != 0, variant, splits, workers, &pc);
    if (rc != SGEMM_OK) return rc;
    if (rows) *rows = pc.rows;
    if (cols) *cols = pc.cols;
    if (first_variant) *first_variant = pc.variant;
    return SGEMM_OK;
}

int sgemm_device_shape(int *compute_units, int *xcds) {
    const Machine m = device_machine();
    if (compute_units) *compute_units = (int)m.cus;
    if (xcds) *xcds = m.xcds;
    return SGEMM_OK;
}

int sgemm_tile_order(int xcds, int nbm, int nbn, int *tile_m, int *tile_n) {
    if (xcds < 1 || xcds > 1024 || (xcds & (xcds - 1)) != 0 || nbm < 0 || nbn < 0 ||
        (long long)nbm * nbn > INT_MAX)
        return SGEMM_ERR_MACHINE;
    if ((long long)nbm * nbn > 0 && (tile_m == nullptr || tile_n == nullptr)) return SGEMM_ERR_MACHINE;
    const int total = nbm * nbn, xs = log2_of(xcds);
    for (int pid = 0; pid < total; ++pid) sgk::tile_of<2, 8>(pid, nbm, nbn, xs, tile_m[pid], tile_n[pid]);
    return SGEMM_OK;
}

int sgemm_select_rows(int M, int N, int K) {
    int rows = 0;
    const int rc = sgemm_select_pieces(M, N, K, &rows, nullptr, nullptr);
    return rc < 0 ? rc : rows;
}

int sgemm_select_pieces(int M, int N, int K, int *rows, int *cols, int *first_variant) {
    if (M < 0) return -1;
    if (N < 0) return -2;
    if (K < 0) return -3;
    const Pieces pc = split_pieces(device_machine(), M, N, K, true);
    if (rows) *rows = pc.rows;
    if (cols) *cols = pc.cols;
    if (first_variant) *first_variant = pc.variant;
    return SGEMM_OK;
}

int sgemm_select_streamk(int M, int N, int K) {
    int w = 0;
    const int rc = plan(device_machine(), M, N, K, true, true, nullptr, nullptr, &w, nullptr);
    return rc < 0 ? rc : w;
}

// Workspace bytes of the plan sgemm_ws makes with enough of it.
size_t plan_bytes(const Machine &m, int M, int N, int K) {
    int v = 0, sp = 1, w = 0;
    if (plan(m, M, N, K, true, true, &v, &sp, &w, nullptr) < 0) return 0;
    if (w > 0) return streamk_bytes(kVariants[v], w);
    return sp > 1 ? splitk_bytes(kVariants[v], sp, M, N) : 0;
}

size_t sgemm_workspace_size(int M, int N, int K) {
    // the plan of operands that allow 16-byte loads (others never split)
    return plan_bytes(device_machine(), M, N, K);
}

int sgemm_ws(int M, int N, int K, float alpha, const float *A, int lda, const float *B,
             int ldb, float beta, float *C, int ldc, void *workspace, size_t workspace_bytes,
             hipStream_t stream) {
    const int rc = check_args(M, N, K, alpha, A, lda, B, ldb, C, ldc);
    if (rc != SGEMM_OK) return rc;
    const Machine m = device_machine();
    int v = 0, sp = 1, w = 0;
    Pieces pc;
    const int prc = plan(m, M, N, K, true, loads16(A, lda, B, ldb, C, ldc), &v, &sp, &w, &pc);
    if (prc != SGEMM_OK) return prc;
    const bool room = workspace != nullptr && ((uintptr_t)workspace & 255u) == 0;
    if (w > 0 || sp > 1) {
        const size_t need = w > 0 ? streamk_bytes(kVariants[v], w) : splitk_bytes(kVariants[v], sp, M, N);
        if (room && workspace_bytes >= need && buffer_offsets_ok(kVariants[v], lda, ldb, ldc))
            return launch(m, v, SGEMM_ACCESS_AUTO, sp, w, workspace, workspace_bytes, M, N, K, alpha, A, lda,
                          B, ldb, beta, C, ldc, stream);
        // not enough workspace: exactly sgemm()
        return sgemm_path(SGEMM_PATH_AUTO, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
    }
    if (pc.rows > 0) return launch_pieces(m, pc, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
    return launch(m, v, SGEMM_ACCESS_AUTO, 1, 0, nullptr, 0, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                  stream);
}

int sgemm_ws_noalloc(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
                     float beta, float *C, int ldc, hipStream_t stream) {
    const int rc = check_args(M, N, K, alpha, A, lda, B, ldb, C, ldc);
    if (rc != SGEMM_OK) return rc;
    const Machine m = device_machine();
    int v = 0, sp = 1, w = 0;
    const int prc = plan(m, M, N, K, true, loads16(A, lda, B, ldb, C, ldc), &v, &sp, &w, nullptr);
    if (prc != SGEMM_OK) return prc;
    // the bytes sgemm_ws would use with enough workspace (none when there is
    // no product to split)
    size_t need = 0;
    if (M > 0 && N > 0 && K > 0 && alpha != 0.0f)
        need = w > 0 ? streamk_bytes(kVariants[v], w) : (sp > 1 ? splitk_bytes(kVariants[v], sp, M, N) : 0);
    if (need > kScratchBytes) return SGEMM_ERR_SCRATCH;
    if (need == 0) return sgemm_ws(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, nullptr, 0, stream);
    const ScratchPtr s = scratch_for_device();
    if (s.ptr == nullptr) return s.err != 0 ? s.err : (int)hipErrorInvalidSymbol;
    // the same plan as sgemm_ws with a workspace of `need` bytes or more
    return sgemm_ws(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s.ptr, kScratchBytes, stream);
}

int sgemm_variant_count(void) { return kNumVariants; }

int sgemm_variant_builds(int variant) {
    if (variant < 0 || variant >= kNumVariants) return SGEMM_ERR_VARIANT;
    const Variant &v = kVariants[variant];
    int bits = SGEMM_BUILD_BUFFER_128 | SGEMM_BUILD_BUFFER_32;
    if (!v.generic_buf) bits |= SGEMM_BUILD_CHECKED;
    if (v.vec4u) bits |= SGEMM_BUILD_BUFFER_128_AB;
    if (v.split4) bits |= SGEMM_BUILD_SPLITK;
    if (v.split4 && v.streamk) bits |= SGEMM_BUILD_STREAMK;
    return bits;
}

#ifdef SGEMM_PHASES
// The phase log of the measurement build (fp32_gemm_03_amd/phases.py): n
// words, 8 per workgroup of the last launch, into host memory.
int sgemm_phase_read(unsigned long long *host, int n) {
    if (host == nullptr || n < 0 || n > sgk::kPhaseWorkgroups * sgk::kPhaseSlots) return SGEMM_ERR_MACHINE;
    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(sgk::sgemm_phase_log), (size_t)n * 8, 0,
                                    hipMemcpyDeviceToHost);
}
#endif

const char *sgemm_variant_name(int variant) {
    if (variant < 0 || variant >= kNumVariants) return nullptr;
    return kVariants[variant].name;
}

int sgemm_variant_path(int variant) {
    if (variant < 0 || variant >= kNumVariants) return SGEMM_ERR_VARIANT;
    return kVariants[variant].path;
}

int sgemm_variant_tile(int variant, int *bm, int *bn) {
    if (variant < 0 || variant >= kNumVariants) return SGEMM_ERR_VARIANT;
    if (bm) *bm = kVariants[variant].bm;
    if (bn) *bn = kVariants[variant].bn;
    return SGEMM_OK;
}

int sgemm_variant_reads_a128(int variant) {
    if (variant < 0 || variant >= kNumVariants) return SGEMM_ERR_VARIANT;
    return kVariants[variant].a128;
}


int sgemm_select_variant(int path, int M, int N, int K) {
    return select_variant(device_machine(), path, M, N, K, true);
}

int sgemm_select_variant_for(int path, int M, int N, int K, const float *A, int lda, const float *B, int ldb,
                             const float *C, int ldc) {
    return select_variant(device_machine(), path, M, N, K, loads16(A, lda, B, ldb, C, ldc));
}

int sgemm_operands_load16(const float *A, int lda, const float *B, int ldb, const float *C, int ldc) {
    return loads16(A, lda, B, ldb, C, ldc) ? 1 : 0;
}

const char *sgemm_status_string(int status) {
    switch (status) {
        case SGEMM_OK: return "success";
        case -1: return "invalid argument: M < 0";
        case -2: return "invalid argument: N < 0";
        case -3: return "invalid argument: K < 0";
        case -5: return "invalid argument: A is NULL";
        case -6: return "invalid argument: lda < max(1, K)";
        case -7: return "invalid argument: B is NULL";
        case -8: return "invalid argument: ldb < max(1, N)";
        case -10: return "invalid argument: C is NULL";
        case -11: return "invalid argument: ldc < max(1, N)";
        case SGEMM_ERR_PATH: return "invalid argument: unknown path";
        case SGEMM_ERR_VARIANT: return "invalid argument: unknown variant";
        case SGEMM_ERR_TOO_LARGE: return "problem too large: tile grid exceeds one launch";
        case SGEMM_ERR_ACCESS: return "invalid argument: access mode unknown or not possible for these arguments";
        case SGEMM_ERR_WORKSPACE: return "invalid argument: workspace missing, too small or not 256-byte aligned";
        case SGEMM_ERR_SPLITS:
            return "invalid argument: split or worker count out of range, or variant without split-K or stream-K";
        case SGEMM_ERR_MACHINE: return "invalid argument: machine shape or tile grid out of range";
        case SGEMM_ERR_SCRATCH:
            return "problem too large for sgemm_ws_noalloc: its plan needs more scratch than the library's static "
                   "buffer holds (use sgemm_ws with a workspace, or sgemm)";
        default: break;
    }
    if (status > 0) return hipGetErrorString((hipError_t)status);
    return "unknown status";
}

int sgemm_device_fp32_peak(int device, int *compute_units, int *clock_khz, double *tflops) {
    hipDeviceProp_t prop;
    const hipError_t e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess) return (int)e;
    // v_mfma_f32_32x32x2_f32: 32*32*2*2 FLOP per 64 cycles on each of 4 SIMDs
    // = 256 FLOP per clock per CU, the same rate as the FP32 vector FMA.
    if (compute_units) *compute_units = prop.multiProcessorCount;
    if (clock_khz) *clock_khz = prop.clockRate;
    if (tflops) *tflops = (double)prop.multiProcessorCount * 256.0 * (double)prop.clockRate * 1e3 / 1e12;
    return SGEMM_OK;
}

}  // extern "C"
