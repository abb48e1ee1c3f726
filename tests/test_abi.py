"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
its host logic (argument checks, variant table, variant choice, status text)
behaves as include/sgemm.h states.  No call here reaches a kernel launch:
argument checks run before any HIP call, and every call below either fails a
check or takes a documented quick return."""
import ctypes
import os
import re

import pytest

import fp32_gemm_03_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgemm.h")


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(sgemm\w*)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("sgemm", "sgemm_path", "sgemm_variant", "sgemm_status_string",
                     "sgemm_variant_count", "sgemm_select_variant"):
        assert required in names, names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(g.library_path())
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_library_has_gfx950_code_object():
    # the shared library carries an offload bundle for gfx950
    blob = open(g.library_path(), "rb").read()
    assert b"gfx950" in blob


def test_no_cpu_fallback_symbols_reference_the_oracle():
    blob = open(g.library_path(), "rb").read()
    assert b"oracle_sgemm" not in blob


def _call(M=4, N=4, K=4, alpha=1.0, A=0x1000, lda=None, B=0x2000, ldb=None,
          beta=0.0, C=0x3000, ldc=None, fn=g.sgemm, path=None, variant=None):
    # The addresses are fake: every call made with them must stop at an
    # argument check or a quick return, never at a launch.
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    lead = () if fn is g.sgemm else ((path,) if fn is g.sgemm_path else (variant,))
    return fn(*lead, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=0, check=False)


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), -1), (dict(N=-1), -2), (dict(K=-1), -3),
    (dict(A=0), -5), (dict(lda=3), -6), (dict(B=0), -7), (dict(ldb=3), -8),
    (dict(C=0), -10), (dict(ldc=3), -11),
    (dict(K=0, lda=0), -6), (dict(N=0, ldb=0, ldc=1), -8),
])
def test_argument_codes(kw, code):
    assert _call(**kw) == code
    assert _call(fn=g.sgemm_path, path=g.SGEMM_PATH_MFMA, **kw) == code
    assert _call(fn=g.sgemm_variant, variant=0, **kw) == code
    assert g.sgemm_status_string(code).startswith("invalid argument")


def test_first_bad_argument_wins():
    assert _call(M=-1, N=-1, lda=0) == -1
    assert _call(A=0, B=0, C=0) == -5


def test_null_operands_allowed_when_not_read():
    # alpha == 0: A and B are not read, beta == 1 leaves C as is: quick return
    assert _call(A=0, B=0, alpha=0.0, beta=1.0) == 0
    # K == 0 and beta == 1: quick return, A and B never read
    assert _call(K=0, lda=1, A=0, B=0, beta=1.0) == 0
    # M == 0 or N == 0: nothing to do, C may be NULL
    assert _call(M=0, C=0, A=0) == 0
    assert _call(N=0, ldb=1, ldc=1, C=0, B=0) == 0


def test_unknown_path_and_variant():
    assert _call(fn=g.sgemm_path, path=7) == -20
    assert _call(fn=g.sgemm_path, path=7, M=0) == -20
    assert _call(fn=g.sgemm_variant, variant=g.sgemm_variant_count(), M=0) == -21
    assert _call(fn=g.sgemm_variant, variant=-1, M=0) == -21
    assert "unknown path" in g.sgemm_status_string(-20)
    assert "unknown variant" in g.sgemm_status_string(-21)


def test_access_mode_codes():
    def acc(mode, **kw):
        base = dict(M=4, N=4, K=4, alpha=1.0, A=0x1000, lda=4, B=0x2000, ldb=4, beta=0.0,
                    C=0x3000, ldc=4)
        base.update(kw)
        return g.sgemm_variant_access(0, mode, *base.values(), stream=0, check=False)
    assert acc(g.SGEMM_ACCESS_BUFFER_128_AB) == -23             # no such build of this variant
    assert acc(5) == -23
    assert acc(-1) == -23
    assert acc(g.SGEMM_ACCESS_BUFFER_128, B=0x2004) == -23     # misaligned B
    assert acc(g.SGEMM_ACCESS_BUFFER_128, N=3, ldb=4, ldc=4) == -23
    assert acc(g.SGEMM_ACCESS_BUFFER_32, lda=1 << 30) == -23    # offsets beyond 31 bits
    assert acc(4, M=-1) == -1                                   # argument checks come first
    assert "access mode" in g.sgemm_status_string(-23)


def test_builds_loading_a_and_b_16_bytes_at_4_byte_alignment():
    """The K-ordered blocks' whole-tile build for rows at 4-byte alignment
    (SGEMM_ACCESS_BUFFER_128_AB): every block the choice takes for large or
    small shapes has one; forcing it needs A, B, C 4-byte aligned and
    in-tile offsets below 2^31 (the refusal comes before any HIP call)."""
    n = g.sgemm_variant_count()
    builds = [g.sgemm_variant_builds(v) for v in range(n)]
    assert g.sgemm_variant_builds(n) == -21 and g.sgemm_variant_builds(-1) == -21
    both = g.SGEMM_BUILD_BUFFER_128 | g.SGEMM_BUILD_BUFFER_32
    assert all(b & both == both for b in builds)
    ua = [v for v in range(n) if builds[v] & g.SGEMM_BUILD_BUFFER_128_AB]
    assert ua and all(g.sgemm_variant_reads_a128(v) == 1 for v in ua)
    # split builds match the split queries; the checked build uses plain
    # pointers except on the small blocks
    for v in range(n):
        assert bool(builds[v] & g.SGEMM_BUILD_SPLITK) == g.variant_has_splitk(v)
        assert bool(builds[v] & g.SGEMM_BUILD_STREAMK) == g.variant_has_streamk(v)
        small = g.sgemm_variant_tile(v)[1] == 32
        assert bool(builds[v] & g.SGEMM_BUILD_CHECKED) == (not small), g.sgemm_variant_name(v)
    for shape in [(256, 256, 256), (1000, 1023, 999), (1024, 1024, 1024), (2048, 2048, 2048),
                  (8192, 8192, 8192), (16384, 16384, 128), (1408, 1408, 1408)]:
        assert g.sgemm_select_variant(g.SGEMM_PATH_AUTO, *shape) in ua, shape
    v = g.sgemm_select_variant(g.SGEMM_PATH_AUTO, 8192, 8192, 8192)

    def acc(**kw):
        base = dict(M=4, N=4, K=4, alpha=1.0, A=0x1000, lda=4, B=0x2000, ldb=4, beta=0.0,
                    C=0x3000, ldc=4)
        base.update(kw)
        return g.sgemm_variant_access(v, g.SGEMM_ACCESS_BUFFER_128_AB, *base.values(), stream=0,
                                      check=False)
    assert acc(A=0x1002) == -23          # A not 4-byte aligned
    assert acc(B=0x2001) == -23
    assert acc(C=0x3003) == -23
    assert acc(lda=1 << 24) == -23       # a tile's rows of A beyond 2^31 bytes
    assert acc(K=0, lda=4, beta=1.0) == 0  # no product: quick return before any launch


def test_variants_reading_a_128_bits_need_k_and_a_aligned():
    """The K-ordered blocks' 128-bit build also reads A 128 bits at a time
    along K, so forcing it needs K, lda multiples of 4 and A 16-byte aligned
    (the refusal comes before any HIP call)."""
    a128 = [v for v in range(g.sgemm_variant_count()) if g.sgemm_variant_reads_a128(v) == 1]
    assert a128 and all(g.sgemm_variant_reads_a128(v) == 0
                        for v in range(g.sgemm_variant_count()) if v not in a128)
    assert all("_kcd" in g.sgemm_variant_name(v) for v in a128)
    assert g.sgemm_variant_reads_a128(g.sgemm_variant_count()) == -21
    assert g.sgemm_variant_reads_a128(-1) == -21
    # the automatic choice for large shapes is one of them
    assert g.sgemm_select_variant(g.SGEMM_PATH_AUTO, 8192, 8192, 8192) in a128
    v = a128[0]

    def acc(**kw):
        base = dict(M=4, N=4, K=4, alpha=1.0, A=0x1000, lda=4, B=0x2000, ldb=4, beta=0.0,
                    C=0x3000, ldc=4)
        base.update(kw)
        return g.sgemm_variant_access(v, g.SGEMM_ACCESS_BUFFER_128, *base.values(), stream=0,
                                      check=False)
    assert acc(K=3, lda=4) == -23        # K not a multiple of 4
    assert acc(K=4, lda=5) == -23        # lda not a multiple of 4
    assert acc(A=0x1004) == -23          # A not 16-byte aligned
    assert acc(K=0, lda=4, beta=1.0) == 0  # no product: quick return before any launch


def test_variant_table():
    vs = g.variants()
    assert len(vs) == g.sgemm_variant_count() >= 2
    paths = {v[2] for v in vs}
    assert paths == {g.SGEMM_PATH_VALU, g.SGEMM_PATH_MFMA}
    for idx, name, path, bm, bn in vs:
        assert name and (name.startswith("valu_") if path == g.SGEMM_PATH_VALU else name.startswith("mfma_"))
        assert bm > 0 and bn > 0 and bm % 32 == 0 and bn % 32 == 0
    assert g.sgemm_variant_name(len(vs)) is None
    assert g.sgemm_variant_path(len(vs)) == -21
    assert g.sgemm_variant_tile(len(vs))[0] == -21


def test_select_variant_is_a_function_of_the_sizes():
    for M, N, K in [(256, 256, 256), (1000, 1023, 999), (1024, 1024, 1024), (4096, 4096, 4096),
                    (8192, 8192, 8192), (16384, 16384, 128), (1, 1, 1)]:
        v = g.sgemm_select_variant(g.SGEMM_PATH_AUTO, M, N, K)
        assert 0 <= v < g.sgemm_variant_count()
        assert g.sgemm_variant_path(v) == g.SGEMM_PATH_MFMA
        assert v == g.sgemm_select_variant(g.SGEMM_PATH_MFMA, M, N, K)
        vv = g.sgemm_select_variant(g.SGEMM_PATH_VALU, M, N, K)
        assert g.sgemm_variant_path(vv) == g.SGEMM_PATH_VALU
    # large squares take the largest tile, and it still fills 256 compute units
    v = g.sgemm_select_variant(0, 8192, 8192, 8192)
    _, bm, bn = g.sgemm_variant_tile(v)
    assert (8192 // bm) * (8192 // bn) >= 256
    assert g.sgemm_select_variant(0, -1, 4, 4) == -1
    assert g.sgemm_select_variant(9, 4, 4, 4) == -20


def test_large_shapes_pick_the_block_whose_last_round_is_fullest():
    """Once a block shape has a tile for every workgroup slot on the chip, the
    choice weighs each block's full-chip rate by how full its last round over
    256 CUs is; short K leaves out the blocks that run one workgroup per CU."""
    def block(M, N, K):
        v = g.sgemm_select_variant(g.SGEMM_PATH_AUTO, M, N, K)
        _, bm, bn = g.sgemm_variant_tile(v)
        bk = int(g.sgemm_variant_name(v).split("_")[1].split("x")[2])
        return bm, bn, bk
    assert block(8192, 8192, 8192) == (256, 256, 32)    # 1024 blocks of 256 x 256: 4 per CU
    assert block(4096, 4096, 4096) == (256, 256, 32)    # 256: 1 per CU
    assert block(16384, 1024, 1024) == (256, 256, 32)   # 256
    assert block(16384, 16384, 128) == (128, 256, 16)   # short K: one-per-CU blocks left out
    assert block(6144, 6144, 6144) == (128, 128, 16)    # 576 of 256 x 256 would leave 1/4 idle
    assert block(7168, 7168, 7168) == (128, 128, 16)
    assert block(10240, 10240, 10240) == (128, 128, 16)
    assert block(1024, 8192, 8192) == (128, 256, 32)    # 256 blocks: one per CU
    assert block(2048, 2048, 2048) == (128, 128, 64)    # 256 blocks: one per CU
    assert "_w8_" in g.sgemm_variant_name(g.sgemm_select_variant(g.SGEMM_PATH_AUTO, 2048, 2048, 2048))
    assert block(3072, 3072, 3072) == (64, 64, 32)      # 128 x 128 would leave 1/4 of a round
    assert block(5120, 5120, 5120) == (64, 64, 32)      # whole rounds of 64 x 64, 6.25 of 128 x 128
    # too few tiles for any slot count (operands that allow 16-byte loads):
    # up to three 32 x 32 tiles per CU, the 32 x 32 block in four
    # wave groups; up to one 64 x 64 tile per CU, the 32 x 64 block in two
    assert block(256, 256, 256) == (32, 32, 64)
    assert block(512, 512, 8192) == (32, 32, 64)
    # with half a 32 x 32 tile to one per CU and K >= 2048, its three-stage
    # ring; with a workspace that one beats split-K only when a part would
    # be shorter than 512 of K
    ring = g.sgemm_select_variant(g.SGEMM_PATH_AUTO, 512, 512, 8192)
    assert g.sgemm_variant_name(ring).endswith("_s3_kcd")
    assert g.sgemm_select_variant(g.SGEMM_PATH_AUTO, 384, 384, 2048) == ring   # 144 tiles
    assert g.sgemm_select_variant(g.SGEMM_PATH_AUTO, 256, 256, 4096) != ring   # 64 tiles
    assert g.sgemm_select_variant(g.SGEMM_PATH_AUTO, 512, 512, 1024) != ring   # short K
    assert g.sgemm_select_variant(g.SGEMM_PATH_AUTO, 768, 768, 4096) != ring   # 576 tiles
    assert g.sgemm_ws_plan(512, 512, 2048)[1:3] == (ring, 1)
    assert g.sgemm_ws_plan(512, 512, 4096)[2] == 8
    assert g.sgemm_ws_plan(256, 256, 4096)[2] == 16
    assert block(768, 768, 768) == (32, 32, 64)         # 576 tiles of 32 x 32
    assert block(1024, 1024, 1024) == (32, 64, 64)      # 1024 of 32 x 32, 256 of 64 x 64
    assert block(1000, 1023, 999) == (32, 64, 64)
    assert block(1088, 1024, 1024) == (32, 64, 64)      # 544 of 32 x 64: within one round of 3 per CU
    assert block(1152, 1152, 1152) == (32, 64, 64)
    # up to two 64 x 64 tiles per CU, the 64 x 64 x 64 block; beyond, 64 x 64 x 32
    assert block(1408, 1408, 1408) == (64, 64, 64)
    assert block(2048, 1024, 1024) == (64, 64, 64)
    assert block(1664, 1664, 1664) == (64, 64, 32)
    assert block(1920, 1920, 1920) == (64, 64, 32)
    # with a workspace and long K, stream-K on 64 x 64 x 32 instead
    rc, v, sp, w = g.sgemm_ws_plan(1280, 1280, 4096)
    assert _block(v) == (64, 64, 32) and w == 256
    rc, v, sp, w = g.sgemm_ws_plan(1408, 1408, 1408)
    assert _block(v) == (64, 64, 64) and (sp, w) == (1, 0)
    # operands at 4-byte alignment take the same blocks (their 16-byte loads
    # of A and B need no more); only in-tile offsets beyond 31 bits keep the
    # 64 x 64 block, whose checked build uses plain pointers
    def block_for(M, N, K, lda, ldb, ldc, off=0):
        v = g.sgemm_select_variant_for(g.SGEMM_PATH_AUTO, M, N, K, 0x10000 + off, lda, 0x20000, ldb,
                                       0x30000, ldc)
        return _block(v)
    assert block_for(1000, 1023, 999, 999, 1023, 1023) == (32, 64, 64)
    assert block_for(1024, 1024, 1024, 1024, 1024, 1024) == (32, 64, 64)
    assert block_for(1024, 1024, 1024, 1024, 1024, 1024, off=4) == (32, 64, 64)   # A not 16-byte aligned
    assert block_for(512, 512, 512, 513, 512, 512) == (32, 32, 64)                # lda not a multiple of 4
    assert block_for(512, 512, 512, 512, 512, 512) == (32, 32, 64)
    assert block_for(512, 512, 512, 1 << 24, 512, 512) == (64, 64, 64)            # 33 rows of A beyond 2^31 bytes
    assert block_for(8192, 8192, 8192, 8192, 8192, 8192) == block(8192, 8192, 8192)
    assert block_for(8191, 8191, 8191, 8191, 8191, 8191) == block(8192, 8192, 8192)


def test_streamk_host_logic():
    sk = [v for v in range(g.sgemm_variant_count()) if g.variant_has_streamk(v)]
    assert sk and all(g.variant_has_splitk(v) for v in sk)
    v = sk[0]
    _, bm, bn = g.sgemm_variant_tile(v)
    assert g.sgemm_streamk_workspace_size(v, 256) == 256 * 2 * bm * bn * 4
    assert g.sgemm_streamk_workspace_size(v, 0) == 0
    assert g.sgemm_streamk_workspace_size(v, 4097) == 0
    assert all(g.sgemm_streamk_workspace_size(w, 256) == 0
               for w in range(g.sgemm_variant_count()) if w not in sk)
    # sgemm_ws shares K tiles where the last round of tiles leaves slots idle
    for M, N, K in [(5120, 5120, 5120), (7168, 7168, 7168), (3072, 3072, 3072)]:
        w = g.sgemm_select_streamk(M, N, K)
        assert w > 0 and w % 256 == 0, (M, N, K, w)
        assert g.sgemm_select_splits(M, N, K) == 1
        assert g.sgemm_workspace_size(M, N, K) > 0
    # below the blocks that fill the chip: one worker per CU evens out the K
    # tiles per CU when the 64 x 64 tiles do not divide evenly over the CUs
    assert g.sgemm_select_streamk(1536, 1536, 1536) == 256
    # whole rounds, short K, one tile per CU and small shapes do not
    for M, N, K in [(8192, 8192, 8192), (4096, 4096, 4096), (16384, 16384, 128), (1024, 1024, 1024),
                    (512, 512, 8192), (768, 768, 768)]:
        assert g.sgemm_select_streamk(M, N, K) == 0, (M, N, K)
    assert g.sgemm_select_streamk(-1, 4, 4) == -1
    # the plan agrees with the single-number queries
    for M, N, K in [(5120, 5120, 5120), (8192, 8192, 8192), (512, 512, 8192), (1000, 1023, 999)]:
        rc, pv, psp, pw = g.sgemm_ws_plan(M, N, K)
        assert rc == 0 and 0 <= pv < g.sgemm_variant_count()
        assert psp == g.sgemm_select_splits(M, N, K) and pw == g.sgemm_select_streamk(M, N, K)
        assert not (psp > 1 and pw > 0)
        if pw == 0 and psp == 1:
            assert pv == g.sgemm_select_variant(g.SGEMM_PATH_AUTO, M, N, K)
    assert g.sgemm_ws_plan(4, -1, 4)[0] == -2

    def call(variant, workers, ws=0x10000, nbytes=1 << 30):
        # fake addresses: every call here must stop at a check before any launch
        return g.sgemm_streamk(variant, workers, 300, 260, 1030, 1.0, 0x1000, 1032, 0x2000, 260,
                               0.0, 0x3000, 260, workspace=ws, workspace_bytes=nbytes, stream=0,
                               check=False)
    assert call(v, 0) == -25
    assert call(v, 4097) == -25
    non_sk = [w for w in range(g.sgemm_variant_count()) if w not in sk][0]
    assert call(non_sk, 3) == -25
    assert call(v, 3, ws=0) == -24                      # missing workspace
    assert call(v, 3, nbytes=16) == -24                 # too small
    assert call(v, 3, ws=0x10010) == -24                # not 256-byte aligned
    # operands without 16-byte loads (A not 4-byte aligned): no split build
    assert g.sgemm_streamk(v, 3, 300, 260, 1030, 1.0, 0x1002, 1032, 0x2000, 260, 0.0, 0x3000, 260,
                           workspace=0x10000, workspace_bytes=1 << 30, stream=0, check=False) == -23


def test_pieces_host_logic():
    """Without a workspace, a partial last round of tiles is avoided by
    cutting C into pieces: a first piece at the top left whose tiles fill
    their rounds (7168^3: 28 x 27 = 756 tiles of 256 x 256, 2.95 rounds of
    256), then the columns right of it, then the rows below it.  The first
    piece runs on the 256 x 256 block, or on 128 x 256 or 128 x 128 tiles
    where that gives no cut and K >= 1536.  Whole rounds, a gain under 2%
    once each tile's start is priced (13824^3), K below 1024 and small shapes
    keep one launch."""
    blocks = {15: (256, 256), 10: (128, 256), 12: (128, 128)}
    for M, N, K, rows, cols, v in [(7168, 7168, 7168, 7168, 6912, 15), (9216, 9216, 9216, 8192, 8192, 15),
                                   (5120, 5120, 5120, 4096, 4096, 15), (4300, 4301, 2048, 4096, 4096, 15),
                                   (8256, 2047, 2048, 8192, 2047, 15), (65536, 300, 4096, 65536, 256, 15),
                                   (5376, 3328, 3072, 4992, 3328, 10), (4608, 3072, 4096, 4096, 1024, 12),
                                   (2946, 2901, 2048, 2944, 2816, 12), (4122, 2098, 1536, 4096, 2048, 10)]:
        got = g.sgemm_select_pieces(M, N, K)
        assert got == (0, rows, cols, v), (M, N, K, got)
        assert g.sgemm_select_rows(M, N, K) == rows
        bm, bn = blocks[v]
        assert g.sgemm_variant_tile(v)[1:] == (bm, bn)
        t = (rows // bm) * -(-cols // bn)
        assert t >= 256 and t / (-(-t // 256) * 256) >= 0.96  # busy share of the rounds
    for M, N, K in [(8192, 8192, 8192), (4096, 4096, 4096), (16384, 16384, 16384), (6144, 6144, 6144),
                    (12288, 12288, 12288), (13824, 13824, 13824), (16384, 16384, 128),
                    (1024, 8192, 8192), (1000, 1023, 999),
                    (256, 256, 256), (0, 8192, 8192), (8192, 0, 8192), (8192, 8192, 0),
                    (8872, 10147, 512), (7926, 6380, 512), (11083, 5078, 1024), (4608, 3072, 1024)]:
        assert g.sgemm_select_pieces(M, N, K) == (0, 0, 0, -1), (M, N, K)
        assert g.sgemm_select_rows(M, N, K) == 0, (M, N, K)
    for M in range(512, 20000, 509):
        for N in (3000, 7168, 11000):
            for K in (1536, 4096):
                rc, r, c, v = g.sgemm_select_pieces(M, N, K)
                assert rc == 0
                if r == 0:
                    assert (c, v) == (0, -1)
                    continue
                # the first piece: whole tiles inside C, or every column
                bm, bn = blocks[v]
                assert r % bm == 0 and 0 < r <= M, (M, N, r, c)
                assert c == N or (c % bn == 0 and 0 < c < N), (M, N, r, c)
                assert (r, c) != (M, N), (M, N)
                assert v == 15 or K >= 1536
    for bad, code in [((-1, 4, 4), -1), ((4, -1, 4), -2), ((4, 4, -1), -3)]:
        assert g.sgemm_select_rows(*bad) == code
        assert g.sgemm_select_pieces(*bad)[0] == code


def test_only_the_latency_block_splits_k():
    """A block chosen by rate already has a tile per workgroup slot on the
    chip; only the 64 x 64 fallbacks split K when a workspace is given."""
    assert g.sgemm_select_splits(1024, 8192, 8192) == 1
    assert g.sgemm_select_splits(2048, 2048, 2048) == 1
    assert g.sgemm_select_splits(16384, 1024, 1024) == 1
    assert g.sgemm_workspace_size(1024, 8192, 8192) == 0


def test_status_strings():
    assert g.sgemm_status_string(0) == "success"
    assert "too large" in g.sgemm_status_string(-22)
    assert g.sgemm_status_string(-999) == "unknown status"


def test_python_binding_raises_on_error():
    with pytest.raises(g.SgemmError) as e:
        g.sgemm(-1, 4, 4, 1.0, 0x1000, 4, 0x2000, 4, 0.0, 0x3000, 4, stream=0)
    assert e.value.status == -1


def test_python_binding_rejects_cpu_tensors():
    import torch
    a = torch.zeros(4, 4)
    with pytest.raises(TypeError):
        g.sgemm(4, 4, 4, 1.0, a, 4, a, 4, 0.0, a, 4, stream=0)


def test_splitk_host_logic():
    split_variants = [v for v in range(g.sgemm_variant_count()) if g.variant_has_splitk(v)]
    assert split_variants, "no variant has a split-K build"
    v = split_variants[0]
    _, bm, bn = g.sgemm_variant_tile(v)
    M, N = 3 * bm + 1, 2 * bn
    tiles = 4 * 2
    ws = g.sgemm_splitk_workspace_size(v, 4, M, N)
    assert ws >= 4 * tiles * bm * bn * 4 and ws % 256 == 0
    assert g.sgemm_splitk_workspace_size(v, 1, M, N) == 0
    assert g.sgemm_splitk_workspace_size(v, 0, M, N) == 0
    assert g.sgemm_splitk_workspace_size(v, 65, M, N) == 0
    for nv in range(g.sgemm_variant_count()):
        if nv not in split_variants:
            assert g.sgemm_splitk_workspace_size(nv, 2, M, N) == 0
    # large shapes fill the chip with tiles: no split, no workspace
    assert g.sgemm_select_splits(8192, 8192, 8192) == 1
    assert g.sgemm_workspace_size(8192, 8192, 8192) == 0
    # few tiles and a deep K split: 4 parts or more of the 64 x 64 block beat
    # the small blocks; 2 or 3 do not; shallow K does not split
    assert g.sgemm_select_splits(512, 512, 8192) == 8
    assert g.sgemm_workspace_size(512, 512, 8192) > 0
    assert g.sgemm_select_splits(1024, 1024, 4096) == 1
    assert g.sgemm_workspace_size(1024, 1024, 4096) == 0
    # operands that allow no 16-byte loads never split (loading 4 bytes per
    # lane into LDS, split launches are slower than whole tiles staged
    # through registers); rows at 4-byte alignment split as 128-bit ones do
    assert g.sgemm_plan_for(256, 512, 512, 8192, True, operands_load16=False)[2] == 1
    assert g.sgemm_plan_for(256, 1536, 1536, 1536, True, operands_load16=False)[3] == 0
    assert g.sgemm_plan_for(256, 1536, 1536, 1536, True)[3] == 256
    v = g.sgemm_ws_plan(511, 511, 8191)[1]

    def ws_plan_for(M, N, K, lda, ldb, ldc, A=0x10000, B=0x20000, C=0x30000):
        return g.sgemm_plan_for(256, M, N, K, True, g.sgemm_operands_load16(A, lda, B, ldb, C, ldc))
    assert ws_plan_for(511, 511, 8191, 8191, 511, 511)[1:3] == (v, g.sgemm_select_splits(511, 511, 8191))
    assert ws_plan_for(511, 511, 8191, 8191, 511, 511, A=0x10002)[2] == 1
    assert g.sgemm_select_splits(1024, 1024, 1024) == 1
    assert g.sgemm_select_splits(256, 256, 256) == 1
    # fewer tiles than CUs: parts may be as short as 256 of K
    assert g.sgemm_select_splits(768, 768, 768) == 1
    assert g.sgemm_select_splits(256, 256, 4096) == 16
    assert _block(g.sgemm_ws_plan(256, 256, 4096)[1]) == (64, 64, 64)
    assert g.sgemm_select_splits(-1, 4, 4) == -1


def test_splitk_argument_codes():
    split_v = [v for v in range(g.sgemm_variant_count()) if g.variant_has_splitk(v)][0]
    plain_v = [v for v in range(g.sgemm_variant_count()) if not g.variant_has_splitk(v)][0]
    base = (64, 64, 64, 1.0, 0x1000, 64, 0x2000, 64, 0.0, 0x3000, 64)

    def call(variant, splits, ws=0x10000, nbytes=1 << 30):
        return g.sgemm_splitk(variant, splits, *base, workspace=ws, workspace_bytes=nbytes,
                              stream=0, check=False)
    assert call(split_v, 0) == -25
    assert call(split_v, 65) == -25
    assert call(plain_v, 2) == -25
    assert call(split_v, 2, ws=0) == -24               # missing workspace
    assert call(split_v, 2, nbytes=16) == -24          # too small
    assert call(split_v, 2, ws=0x10010) == -24         # not 256-byte aligned
    # operands without 16-byte loads (B not 4-byte aligned): no split build
    assert g.sgemm_splitk(split_v, 2, 64, 64, 64, 1.0, 0x1000, 64, 0x2002, 64, 0.0, 0x3000, 64,
                          workspace=0x10000, workspace_bytes=1 << 30, stream=0, check=False) == -23
    assert "workspace" in g.sgemm_status_string(-24)
    assert "split" in g.sgemm_status_string(-25)


def test_grid_too_large_is_refused_before_any_hip_call():
    # 2^31 - 1 square: tiles of every variant number far more than INT_MAX, so
    # the launch is refused with SGEMM_ERR_TOO_LARGE before anything touches
    # the (never dereferenced) pointers or a GPU
    big = 2 ** 31 - 1
    args = (big, big, 1, 1.0, 256, 1, 256, big, 0.0, 256, big)
    assert g.sgemm(*args, stream=0, check=False) == -22
    assert g.sgemm_path(g.SGEMM_PATH_VALU, *args, stream=0, check=False) == -22
    for v in range(g.sgemm_variant_count()):
        assert g.sgemm_variant(v, *args, stream=0, check=False) == -22, v



def test_device_shape_and_plan_for_256_cus():
    """Without a GPU the library plans for an MI355X (256 CUs, 8 XCDs), and
    the explicit-shape plan at 256 CUs is exactly what the device queries
    return, with and without a workspace."""
    cus, xcds = g.sgemm_device_shape()
    assert cus > 0 and xcds >= 1 and xcds & (xcds - 1) == 0
    import torch
    if not torch.cuda.is_available():
        assert (cus, xcds) == (256, 8)
    shapes = [(256, 256, 256), (1000, 1023, 999), (1024, 1024, 1024), (2048, 2048, 2048),
              (4096, 4096, 4096), (8192, 8192, 8192), (16384, 16384, 128), (5120, 5120, 5120),
              (7168, 7168, 7168), (13824, 13824, 13824), (512, 512, 8192), (1536, 1536, 1536),
              (40000, 300, 4096), (1, 1, 1), (0, 5, 5)]
    for M, N, K in shapes:
        rc, v, sp, w, rows = g.sgemm_plan_for(cus, M, N, K)
        assert rc == 0 and sp == 1 and w == 0
        assert v == g.sgemm_select_variant(g.SGEMM_PATH_AUTO, M, N, K), (M, N, K)
        assert rows == g.sgemm_select_rows(M, N, K), (M, N, K)
        assert g.sgemm_plan_pieces_for(cus, M, N, K) == (rc, v, sp, w) + g.sgemm_select_pieces(M, N, K)[1:]
        rc, v2, sp2, w2, rows2 = g.sgemm_plan_for(cus, M, N, K, with_workspace=True)
        assert (rc, v2, sp2, w2) == g.sgemm_ws_plan(M, N, K), (M, N, K)
        assert sp2 == g.sgemm_select_splits(M, N, K) and w2 == g.sgemm_select_streamk(M, N, K)
        assert rows2 == (g.sgemm_select_rows(M, N, K) if (sp2, w2) == (1, 0) else 0)
    assert g.sgemm_plan_for(0, 4, 4, 4)[0] == -26
    assert g.sgemm_plan_for(256, -1, 4, 4)[0] == -1
    assert g.sgemm_plan_for(256, 4, 4, -1)[0] == -3
    assert "machine shape" in g.sgemm_status_string(-26)


def _block(v):
    _, bm, bn = g.sgemm_variant_tile(v)
    bk = int(g.sgemm_variant_name(v).split("_")[1].split("x")[2])
    return bm, bn, bk


def _last_round_busy(tiles, cus):
    return tiles / (-(-tiles // cus) * cus)


@pytest.mark.parametrize("cus", [32, 80])
def test_plan_quantises_over_other_cu_counts(cus):
    """On a device with another CU count (a one-XCD partition of 32 CUs, or
    80) the same rates are weighed against that count: the chosen block has a
    tile for every one of its workgroup slots or is the latency block, its
    last round keeps most CUs busy, stream-K takes one worker per CU and
    split-K aims at about two workgroups per CU."""
    per_cu = {"_w16_kcd": 1, "x32_w128x64_kcd": 1, "_wpe4_kcd": 4, "x16_w64x128_kcd": 2,
              "x32_w64x64_w8_kcd": 1, "64x64x32_w32x32_kcd": 4, "x64_w32x64_w8_kcd": 1,
              "_kg2_kcd": 2, "_kg4_kcd": 4, "x32_w64x32_w8_kcd": 2}
    fallbacks = ("mfma_64x64x64_w64x32_kg2_kcd", "mfma_64x64x32_w32x32_kcd",
                 "mfma_32x32x64_w32x32_kg4_kcd", "mfma_32x64x64_w32x32_kg2_kcd")
    for M, N, K in [(8192, 8192, 8192), (4096, 4096, 4096), (2048, 2048, 2048), (1024, 1024, 1024),
                    (6144, 6144, 6144), (16384, 16384, 128), (3000, 5000, 2000)]:
        rc, v, sp, w, rows = g.sgemm_plan_for(cus, M, N, K)
        assert rc == 0 and g.sgemm_variant_path(v) == g.SGEMM_PATH_MFMA
        bm, bn, _ = _block(v)
        name = g.sgemm_variant_name(v)
        t = -(-M // bm) * -(-N // bn)
        slots = [n for k, n in per_cu.items() if name.endswith(k)]
        assert slots, name
        if name not in fallbacks:
            assert t >= slots[0] * cus, (cus, M, N, K, name)
        if t >= 4 * cus and rows == 0:
            assert _last_round_busy(t, cus) >= 0.8, (cus, M, N, K, name, t)
        rc, v2, sp2, w2, _ = g.sgemm_plan_for(cus, M, N, K, with_workspace=True)
        assert w2 in (0, cus)
        if sp2 > 1:
            bm2, bn2, _ = _block(v2)
            t2 = -(-M // bm2) * -(-N // bn2)
            assert t2 <= cus and t2 * sp2 <= 2 * cus
    # a 32-CU partition fills its CUs with 128 x 256 blocks at 1024^3, where
    # 256 CUs need a small block (32 x 64; 64 x 64 for operands that allow
    # no 16-byte loads)
    assert _block(g.sgemm_plan_for(32, 1024, 1024, 1024)[1])[:2] == (128, 256)
    assert _block(g.sgemm_plan_for(256, 1024, 1024, 1024)[1])[:2] == (32, 64)
    assert _block(g.sgemm_plan_for(256, 1024, 1024, 1024, operands_load16=True)[1])[:2] == (32, 64)
    assert _block(g.sgemm_plan_for(256, 1024, 1024, 1024, operands_load16=False)[1])[:2] == (64, 64)
    # split-K: 64 tiles of 64 x 64 at 512 x 512 x 8192 split in 8 on 256 CUs;
    # on 80 CUs a split would be in 2, so the 32 x 64 block runs whole
    # instead; operands without 16-byte loads neither split nor take it
    assert g.sgemm_plan_for(256, 512, 512, 8192, True)[2] == 8
    assert g.sgemm_plan_for(80, 512, 512, 8192, True)[2] == 1
    assert _block(g.sgemm_plan_for(80, 512, 512, 8192, True)[1])[:2] == (32, 64)
    assert g.sgemm_plan_for(80, 512, 512, 8192, True, operands_load16=False)[2] == 1
    assert _block(g.sgemm_plan_for(80, 512, 512, 8192, True, operands_load16=False)[1])[:2] == (64, 64)


def test_tile_order_is_a_bijection_for_every_xcd_count():
    """Workgroup -> tile order of the K-ordered blocks: every tile exactly
    once for 1, 2, 4 and 8 XCDs on every grid up to 24 x 24 (and a few
    larger); row-major when the tile columns divide evenly over the XCDs or
    there is one XCD; otherwise XCD x (workgroups x, x + X, ...) keeps its own
    columns x, x + X, ... until the remainder columns."""
    grids = [(a, b) for a in range(1, 25) for b in range(1, 25)] + [(3, 11), (32, 54), (69, 69), (1, 200)]
    for X in (1, 2, 4, 8):
        for nbm, nbn in grids:
            rc, tm, tn = g.sgemm_tile_order(X, nbm, nbn)
            assert rc == 0
            seen = set(zip(tm, tn))
            assert len(seen) == nbm * nbn and seen == {(m, n) for m in range(nbm) for n in range(nbn)}, \
                (X, nbm, nbn)
            if X == 1 or nbn % X == 0 or nbn < X:
                assert tm == [p // nbn for p in range(nbm * nbn)] and tn == [p % nbn for p in range(nbm * nbn)]
            else:
                own = nbm * (nbn // X)  # tiles each XCD takes in its own columns
                for p in range(X * own):
                    assert tn[p] % X == p % X and tn[p] < X * (nbn // X), (X, nbm, nbn, p)
    assert g.sgemm_tile_order(3, 2, 2)[0] == -26   # not a power of two
    assert g.sgemm_tile_order(0, 2, 2)[0] == -26
    assert g.sgemm_tile_order(8, -1, 2)[0] == -26
    assert g.sgemm_tile_order(8, 0, 5) == (0, [], [])


@pytest.mark.parametrize("cus", [32, 80, 256, 304])
def test_pieces_tile_c_on_any_cu_count(cus):
    """On any CU count, a cut's first piece is whole tiles of its block (or
    every column, padded) inside C and not all of it, its tiles fill at least
    96% of their last round of that many CUs, and only K >= 1024 is cut.
    Random shapes, seeded."""
    import numpy as np
    blocks = {15: (256, 256), 10: (128, 256), 12: (128, 128)}
    rng = np.random.default_rng(cus)
    taken = 0
    for _ in range(400):
        M, N = (int(x) for x in rng.integers(256, 20000, 2))
        K = int(rng.choice([512, 1024, 1536, 2048, 4096, 8192]))
        rc, v, sp, w, rows, cols, first = g.sgemm_plan_pieces_for(cus, M, N, K)
        assert rc == 0 and sp == 1 and w == 0
        if rows == 0:
            assert (cols, first) == (0, -1)
            continue
        taken += 1
        assert first in blocks and K >= 1024, (M, N, K, first)
        bm, bn = blocks[first]
        assert rows % bm == 0 and 0 < rows <= M
        assert cols == N or (cols % bn == 0 and 0 < cols < N)
        assert (rows, cols) != (M, N)
        t = (rows // bm) * -(-cols // bn)
        assert t >= cus and t / (-(-t // cus) * cus) >= 0.96, (M, N, K, rows, cols, t)
    assert taken > 0


def test_narrow_n_weighs_the_tiles_area_inside_c():
    """Padded tile columns still issue every MFMA: with N = 260 or 300 a
    256-wide block is 51-59% inside C, a 64 x 64 block 81-94%, and the
    choice follows that share.  A cut into pieces never pads a wide first
    piece here: it takes the first 256 (or 128) columns alone where their
    tiles fill whole rounds (65536 rows: 256 tiles of 256 x 256; 32768 rows:
    256 of 128 x 128), the rest of the columns going to a second launch.
    Measured against one launch: 65536 x 300 x 4096 130.5 against 116.7
    TFLOP/s, 40000 x 300 x 4096 112.0 against 106.8."""
    for M, N, K, cut in [(40000, 300, 4096, (32768, 128, 12)), (65536, 260, 4096, (65536, 256, 15)),
                         (40000, 260, 4096, (32768, 128, 12)), (16384, 300, 4096, None),
                         (65536, 300, 4096, (65536, 256, 15))]:
        v = g.sgemm_select_variant(g.SGEMM_PATH_AUTO, M, N, K)
        bm, bn, _ = _block(v)
        fill = M * N / (-(-M // bm) * bm * -(-N // bn) * bn)
        assert bn == 64 and fill >= 0.8, (M, N, K, g.sgemm_variant_name(v), fill)
        assert g.sgemm_select_pieces(M, N, K) == ((0,) + cut if cut else (0, 0, 0, -1)), (M, N, K)
        if cut:
            rows, cols, _ = cut
            v2 = g.sgemm_select_variant(g.SGEMM_PATH_AUTO, rows, N - cols, K)
            assert _block(v2)[1] == 64, g.sgemm_variant_name(v2)
    # wide N keeps the 256 x 256 block and the cut where they fill C
    assert _block(g.sgemm_select_variant(g.SGEMM_PATH_AUTO, 8192, 8192, 8192))[:2] == (256, 256)
    assert g.sgemm_select_pieces(7168, 7168, 7168) == (0, 7168, 6912, 15)


def test_operands_load16_condition():
    """Operands that allow 16-byte loads of A and B: A, B and C 4-byte
    aligned and in-tile byte offsets of the small blocks below 2^31, whatever
    the leading dimensions are modulo 4 (the pointers are only inspected)."""
    ok = (0x1000, 1024, 0x2000, 1024, 0x3000, 1024)
    assert g.sgemm_operands_load16(*ok)
    for i, fine in [(0, 0x1004), (1, 1021), (2, 0x2008), (3, 1026), (4, 0x300c), (5, 1027)]:
        args = list(ok)
        args[i] = fine
        assert g.sgemm_operands_load16(*args), (i, fine)
    for i, bad in [(0, 0x1002), (1, 1 << 24), (2, 0x2001), (3, 1 << 24), (4, 0x3003), (5, 1 << 24)]:
        args = list(ok)
        args[i] = bad
        assert not g.sgemm_operands_load16(*args), (i, bad)


def test_small_blocks_need_31_bit_offsets():
    """The 32 x 32 and 32 x 64 wave-group blocks have only buffer-access
    builds: leading dimensions too large for 31-bit in-tile offsets keep the
    choice off them, and forcing them is refused before any HIP call."""
    big = 1 << 26   # floats: 33 rows of A span more than 2^31 bytes
    assert not g.sgemm_operands_load16(0x1000, big, 0x2000, 512, 0x3000, 512)
    v = g.sgemm_select_variant_for(g.SGEMM_PATH_AUTO, 512, 512, 512, 0x1000, big, 0x2000, 512, 0x3000, 512)
    assert _block(v) == (64, 64, 64)
    tiny = [i for i in range(g.sgemm_variant_count()) if (g.sgemm_variant_name(i) or "").startswith("mfma_32x")]
    assert len(tiny) == 3   # 32 x 32 (two and three LDS stages) and 32 x 64
    for t in tiny:
        for access in (g.SGEMM_ACCESS_AUTO, g.SGEMM_ACCESS_CHECKED):
            rc = g.sgemm_variant_access(t, access, 512, 512, 512, 1.0, 0x1000, big, 0x2000, 512, 0.0,
                                        0x3000, 512, stream=0, check=False)
            assert rc == -23, (t, access, rc)


def test_no_kernel_uses_scratch():
    """Every kernel in the library keeps its state in registers and LDS: no
    register spills to scratch memory (read from the AMDGPU metadata of the
    built gfx950 code object)."""
    from fp32_gemm_03_amd import build as b
    try:
        res = b.kernel_resources()
    except (RuntimeError, OSError) as e:
        pytest.skip(f"cannot read the code object: {e}")
    assert len(res) >= 3 * g.sgemm_variant_count(), len(res)
    names = dict(zip(res, b.demangle(res)))
    bad = {names[k]: r for k, r in res.items()
           if r.get("private_segment_fixed_size", -1) != 0 or r.get("vgpr_spill_count", -1) != 0}
    assert not bad, bad
    # the LDS each kernel declares fits a CU's 160 KiB
    assert all(0 < r["group_segment_fixed_size"] <= 160 * 1024 for r in res.values())


def test_noalloc_entry_point_checks_before_any_hip_call():
    """sgemm_ws_noalloc validates like sgemm_ws, and refuses a plan whose
    partial tiles exceed its static scratch (stream-K on 256 x 256 tiles of
    7168^3 needs 128 MiB) before touching the (fake) pointers or a GPU."""
    assert g.SGEMM_NOALLOC_SCRATCH_BYTES == 32 << 20
    args = lambda M, N, K: (M, N, K, 1.0, 0x1000, K, 0x2000, N, 0.0, 0x3000, N)
    assert g.sgemm_ws_noalloc(*args(-1, 4, 4), stream=0, check=False) == -1
    assert g.sgemm_ws_noalloc(*args(7168, 7168, 7168), stream=0, check=False) == -27
    assert g.sgemm_workspace_size(7168, 7168, 7168) > g.SGEMM_NOALLOC_SCRATCH_BYTES
    assert "static buffer" in g.sgemm_status_string(-27)
    # quick returns need no scratch and no launch
    assert g.sgemm_ws_noalloc(0, 5, 5, 1.0, 0, 5, 0x2000, 5, 0.0, 0, 5, stream=0, check=False) == 0
    # every split-K plan fits: at most two partial 64 x 64 tiles per CU
    for M, N, K in [(512, 512, 8192), (256, 256, 4096), (64, 64, 16384), (1536, 1536, 1536)]:
        assert 0 < g.sgemm_workspace_size(M, N, K) <= g.SGEMM_NOALLOC_SCRATCH_BYTES, (M, N, K)
