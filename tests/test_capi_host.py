"""The C-ABI library on the CPU: it loads, exports every declared symbol, and its
host-side argument checks answer without touching a GPU."""
import ctypes
import math
import os
import random
import re

import pytest

import linear_algebra_sgemm_amd as lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("gemm.h", "gemm_debug.h")]


def _declared_functions():
    names = []
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\([^;]*\)\s*;", text, flags=re.M)
    return names


@pytest.fixture(scope="module")
def so():
    if not os.path.exists(lib.library_path()):
        pytest.fail("libgemm.so is not built; run __graft_entry__.build() first")
    return lib.load_library()


def test_headers_declare_the_boundary():
    names = set(_declared_functions())
    assert {"gemm_create", "gemm_destroy", "sgemm", "hgemm_bias_act", "bgemm_bias_act",
            "gemm_status_string"} <= names
    assert names == set(lib.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(so):
    for name in _declared_functions():
        assert hasattr(so, name), name
        assert ctypes.cast(getattr(so, name), ctypes.c_void_p).value


def test_status_strings(so):
    for st in range(6):
        assert lib.gemm_status_string(st)
    assert "invalid" in lib.gemm_status_string(lib.STATUS_INVALID_VALUE)


BAD_SGEMM = [
    dict(M=-1), dict(N=-1), dict(K=-1),
    dict(lda=3),            # lda < K
    dict(ldb=4),            # ldb < N
    dict(ldc=4),            # ldc < N
    dict(C=None),
    dict(A=None), dict(B=None),
]


@pytest.mark.parametrize("bad", BAD_SGEMM, ids=lambda d: ",".join("%s=%s" % kv for kv in d.items()))
def test_sgemm_rejects_bad_arguments_without_gpu(so, bad):
    args = dict(M=8, N=5, K=4, alpha=1.0, A=0x1000, lda=4, B=0x2000, ldb=5, beta=0.0, C=0x3000,
                ldc=5)
    args.update(bad)
    st = lib.sgemm(args["M"], args["N"], args["K"], args["alpha"], args["A"], args["lda"],
                   args["B"], args["ldb"], args["beta"], args["C"], args["ldc"], stream=0,
                   raise_on_error=False)
    assert st == lib.STATUS_INVALID_VALUE


def test_sgemm_unread_operands_may_be_null(so):
    # alpha == 0: A and B are not read, so NULL is fine; the call then stops at the
    # missing gemm_create (no GPU here), not at argument validation.
    st = lib.sgemm(8, 5, 4, 0.0, None, 4, None, 5, 2.0, 0x3000, 5, stream=0, raise_on_error=False)
    assert st == lib.STATUS_NOT_INITIALIZED
    st = lib.sgemm(8, 5, 0, 1.0, None, 1, None, 5, 2.0, 0x3000, 5, stream=0, raise_on_error=False)
    assert st == lib.STATUS_NOT_INITIALIZED
    # M == 0: nothing is read or written.
    st = lib.sgemm(0, 5, 4, 1.0, None, 4, None, 5, 0.0, None, 5, stream=0, raise_on_error=False)
    assert st == lib.STATUS_NOT_INITIALIZED


def test_hgemm_rejects_bad_arguments_without_gpu(so):
    ok = dict(M=8, N=16, K=8, alpha=1.0, A=0x1000, lda=8, B=0x2000, ldb=16, bias=None, act=1,
              C=0x3000, ldc=16)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return lib.hgemm_bias_act(a["M"], a["N"], a["K"], a["alpha"], a["A"], a["lda"], a["B"],
                                  a["ldb"], a["bias"], a["act"], a["C"], a["ldc"], stream=0,
                                  raise_on_error=False)

    assert call(act=2) == lib.STATUS_INVALID_VALUE
    b = dict(ok)
    b["act"] = 7
    assert lib.bgemm_bias_act(b["M"], b["N"], b["K"], b["alpha"], b["A"], b["lda"], b["B"],
                              b["ldb"], b["bias"], b["act"], b["C"], b["ldc"], stream=0,
                              raise_on_error=False) == lib.STATUS_INVALID_VALUE
    b["act"] = 1
    assert lib.bgemm_bias_act(b["M"], b["N"], b["K"], b["alpha"], b["A"], b["lda"], b["B"],
                              b["ldb"], b["bias"], b["act"], b["C"], b["ldc"], stream=0,
                              raise_on_error=False) == lib.STATUS_NOT_INITIALIZED
    assert call(act=-1) == lib.STATUS_INVALID_VALUE
    assert call(lda=7) == lib.STATUS_INVALID_VALUE
    assert call(ldc=15) == lib.STATUS_INVALID_VALUE
    assert call(C=None) == lib.STATUS_INVALID_VALUE
    assert call(B=None) == lib.STATUS_INVALID_VALUE
    assert call() == lib.STATUS_NOT_INITIALIZED
    assert call(alpha=0.0, A=None, B=None) == lib.STATUS_NOT_INITIALIZED


def test_destroy_without_create(so):
    assert lib.gemm_destroy(raise_on_error=False) == lib.STATUS_NOT_INITIALIZED


TUNED_TABLE = os.path.join(ROOT, "linear_algebra_sgemm_amd", "csrc", "gemm_tuned.inc")


def tuned_classes():
    """(op, class M, class N, class K) of every entry of the offline-tuned table."""
    out = set()
    for line in open(TUNED_TABLE):
        m = re.match(r"\s*\{\s*(-?\d+)\s*,\s*(\d+)\s*,\s*(\d+)\s*,\s*(\d+)\s*,", line)
        if m:
            out.add(tuple(int(g) for g in m.groups()))
    return out


def size_class(x):
    c = round(math.log2(x)) if x > 1 else 7
    return min(max(c, 7), 14)


def load_raw():
    return lib.load_library()


def pick(op, M, N, K, cus=256):
    return lib.gemm_debug_pick_config(op, M, N, K, cus)


def test_config_rule(so):
    """The built-in rule (tuned table off): the largest tile that still gives every
    CU two tiles, split-K only when the tiles do not cover the CUs."""
    cases = [
        (0, 4096, 4096, 4096, 256, (9, 1)),   # whole 256x256 tiles: direct-to-LDS kernel
        (0, 8192, 8192, 8192, 256, (9, 1)),
        (0, 4096, 4096, 4008, 256, (9, 1)),   # ragged K: the bounds-checked direct-to-LDS kernel
        (0, 4000, 4000, 4000, 256, (9, 1)),   # ragged M, N, K likewise
        (0, 4096, 4096, 4002, 256, (9, 1)),   # lda = 4002: A copied 4 bytes at a time
        (0, 4096, 4090, 4096, 256, (9, 1)),   # N not a multiple of 4: B packed first
        (0, 64, 4090, 64, 256, (13, 1)),      # 1024 tiles of 16x16, short K: any operands, no packing
        (0, 256, 256, 256, 256, (13, 1)),     # 256 tiles of 16x16: one per CU, K in the waves
        (0, 256, 256, 1024, 256, (13, 1)),
        (0, 250, 250, 400, 256, (13, 1)),     # ragged, not packable: still the 16x16 tile
        (0, 60, 2000, 2000, 256, (13, 1)),    # 500 tiles of 16x16: two per CU
        (0, 330, 330, 777, 256, (13, 1)),
        (0, 256, 256, 4096, 256, (13, 1)),    # one 16x16 tile per CU: K up to 4096 in the waves
        (0, 256, 512, 4096, 256, (11, 8)),    # two per CU and K > 2048: 64x64 direct in K chunks
        (0, 128, 128, 8192, 256, (11, 16)),   # K > 4096
        (0, 700, 700, 400, 256, (11, 1)),     # 1936 tiles of 16x16: more than two per CU
        (0, 500, 500, 2000, 256, (11, 3)),    # 64 tiles of 64x64, K > 1024: not the 32x32 tile
        (0, 512, 512, 777, 256, (12, 1)),     # four 16x16 tiles per CU, 512 < K <= 1024: 32x32
        (0, 512, 512, 512, 256, (13, 1)),     # 1024 tiles of 16x16 (four per CU), K <= 512
        (0, 512, 512, 480, 256, (13, 1)),
        (0, 512, 512, 500, 256, (13, 1)),     # K not a multiple of 32
        (0, 512, 576, 512, 256, (11, 1)),     # 72 tiles of 64x64
        (0, 1000, 3000, 777, 256, (11, 1)),   # 752 tiles
        (0, 2048, 2048, 2048, 256, (10, 1)),  # 64 tiles of 256x256, 256 of 128x128: direct 128x128
        (0, 2048, 2048, 8192, 256, (10, 1)),
        (0, 1024, 2048, 4096, 256, (10, 2)),  # 128 tiles of 128x128, 2 chunks of 2048
        (0, 1024, 1024, 4096, 256, (10, 4)),  # 64 tiles, 4 chunks of 1024
        (0, 1024, 1024, 8192, 256, (10, 4)),
        (0, 2048, 4096, 1024, 256, (10, 1)),  # 512 tiles of 128x128
        (0, 512, 512, 8192, 256, (11, 8)),    # 16 tiles of 128x128 only: 64 of 64x64, 8 chunks
        (0, 1024, 3072, 768, 256, (11, 1)),   # 192 tiles of 128x128 would need a split of 1
        (0, 1536, 3072, 2048, 256, (11, 1)),  # 288 tiles of 128x128 fill 56 % of 512 slots
        (0, 1000, 1000, 1000, 256, (11, 1)),  # 256 tiles of 64x64: no split
        (0, 1536, 1536, 6144, 256, (9, 7)),   # 36 tiles of 256x256, long K: 7 chunks
        (0, 777, 7777, 777, 256, (11, 1)),    # 128-row tiles leave 13 % of the last row empty
        (0, 2800, 2800, 2800, 256, (10, 1)),
        (0, 3000, 3000, 3000, 256, (11, 1)),  # 576 tiles of 128x128 use 75 % of 512 slots
        (0, 1280, 1280, 8192, 256, (9, 10)),  # 100 tiles of 128x128 in 2 chunks fill 78 %
        (0, 1792, 1792, 4096, 256, (9, 5)),
        (0, 600, 600, 5000, 256, (11, 5)),    # 100 tiles: about two workgroups per CU
        (0, 4096, 4096, 4096, 64, (9, 1)),
        (0, 128, 128, 16384, 256, (11, 16)),  # 4 tiles; 128 chunks by CUs, capped at 16
        (0, 300, 520, 100, 256, (13, 1)),     # ragged and small: the K-split tile
        (0, 300, 521, 100, 256, (13, 1)),     # N odd: the K-split tile takes any operands
        (1, 4096, 14336, 4096, 256, (7, 1)),  # whole 256-tiles, long K: eight waves + tail split
        (1, 4096, 4096, 4096, 256, (6, 1)),   # no partial round: eight waves, no split
        (1, 4096, 4096, 1024, 256, (6, 1)),   # shorter K: eight waves, no split
        (1, 3072, 3072, 3072, 256, (6, 1)),   # 144 tiles of 256x256, 576 of 128x128
        (1, 4096, 4000, 4096, 256, (6, 1)),   # ragged N: eight waves, no column split
        (1, 4096, 4004, 4096, 256, (6, 1)),   # N not a multiple of 8: B packed first
        (1, 2048, 2000, 4096, 256, (8, 1)),   # ragged N, 256 tiles of 128x128: direct 128x128
        (1, 1000, 1000, 1000, 256, (8, 1)),   # ragged, 64 tiles of 128x128
        (1, 1000, 1004, 1000, 256, (8, 1)),   # N not a multiple of 8: B packed, as above
        (1, 3000, 3000, 3000, 256, (6, 1)),   # 576 tiles of 128x128: more than one round
        (1, 4096, 2048, 4096, 256, (8, 1)),   # 512 tiles of 128x128: one round at two per CU
        (1, 4096, 4096, 256, 256, (6, 1)),    # K = 256: still the eight-wave tile
        (1, 4096, 4096, 64, 256, (1, 1)),     # K < 128: register-staged 128x128
        (1, 300, 500, 4096, 256, (8, 4)),      # 12 tiles of 128x128, K >= 4096: direct, chunks of 1024
        (1, 256, 256, 256, 256, (9, 1)),       # 256 tiles of 16x16: K split over the waves
        (1, 250, 250, 400, 256, (9, 1)),       # ragged, any operands
        (1, 500, 500, 400, 256, (9, 1)),       # 1024 tiles of 16x16, K <= 2048
        (1, 256, 256, 4096, 256, (9, 1)),      # one 16x16 tile per CU, K <= 4096
        (1, 512, 512, 4096, 256, (8, 4)),      # 1024 tiles of 16x16 and K > 2048: 128x128 direct
        (1, 700, 700, 400, 256, (4, 1)),       # 1936 tiles of 16x16: not the K-split tile
        (1, 64, 4096, 2049, 256, (8, 2)),      # 32 tiles of 128x128, K >= 1024: direct, split
        (1, 100, 4096, 3000, 256, (8, 2)),
        (1, 1024, 1024, 4096, 256, (8, 4)),    # 64 tiles of 128x128: direct 128x128 in 4 chunks
        (1, 1024, 1024, 4095, 256, (8, 3)),    # the same with K ragged (A packed: half rows)
        (1, 2048, 1024, 8192, 256, (8, 2)),    # 128 tiles: 2 chunks
        (1, 512, 512, 4096, 256, (8, 4)),      # 16 tiles of 128x128, K >= 4096: 4 chunks of 1024
        (1, 512, 512, 2048, 256, (9, 1)),      # 1024 tiles of 16x16, K <= 2048
        (1, 512, 512, 256, 256, (9, 1)),       # 1024 tiles of 16x16, short K
    ]
    assert lib.gemm_debug_use_tuned_table(False) == lib.STATUS_SUCCESS
    try:
        for op, M, N, K, cus, want in cases:
            assert pick(op, M, N, K, cus) == want, (op, M, N, K, cus)
    finally:
        assert lib.gemm_debug_use_tuned_table(True) == lib.STATUS_SUCCESS
    assert load_raw().gemm_debug_use_tuned_table(2) == lib.STATUS_INVALID_VALUE
    # with the table on, the shapes the table does not list still follow the rule
    table = tuned_classes()
    for op, M, N, K, cus, want in cases:
        if (op, size_class(M), size_class(N), size_class(K)) not in table:
            assert pick(op, M, N, K, cus) == want, (op, M, N, K, cus)


def test_sgemm_direct_tile_resolution(so):
    """The FP32 direct-to-LDS tiles take any M, N, K with N a multiple of 4 (ragged
    edges and K run their bounds-checked instantiation); otherwise tile 4 runs."""
    try:
        assert lib.gemm_debug_force_tile(0, 7) == lib.STATUS_SUCCESS
        assert lib.gemm_debug_force_splits(0, 1) == lib.STATUS_SUCCESS
        assert pick(0, 4096, 4096, 4096) == (7, 1)
        assert pick(0, 4096, 4096, 4008) == (7, 1)      # K not a multiple of 32
        assert pick(0, 4000, 4096, 4096) == (7, 1)      # ragged M
        assert pick(0, 4096, 4090, 4096) == (7, 1)      # N not a multiple of 4: B packed
        assert pick(0, 64, 4090, 64) == (4, 1)          # packing costs more than it saves
        assert lib.gemm_debug_force_splits(0, 4) == lib.STATUS_SUCCESS
        assert pick(0, 256, 256, 4096) == (7, 4)        # the direct-to-LDS tiles split too
        assert pick(0, 300, 260, 1000) == (7, 4)        # chunks of 256, 256, 256, 232
        assert lib.gemm_debug_force_tile(0, 8) == lib.STATUS_SUCCESS
        assert lib.gemm_debug_force_splits(0, 1) == lib.STATUS_SUCCESS
        assert pick(0, 128, 256, 64) == (8, 1)
        assert pick(0, 128, 200, 64) == (8, 1)
        assert pick(0, 128, 201, 64) == (4, 1)
    finally:
        lib.gemm_debug_force_tile(0, -1)
        lib.gemm_debug_force_splits(0, -1)


def test_half_split_legality(so):
    """The half products split only on register-staged tiles, in whole K steps of 64."""
    try:
        assert lib.gemm_debug_force_splits(1, 8) == lib.STATUS_SUCCESS
        assert lib.gemm_debug_force_tile(1, 2) == lib.STATUS_SUCCESS
        assert pick(1, 256, 256, 4096) == (2, 8)       # 64 K steps, 8 per chunk
        assert pick(1, 256, 256, 200) == (2, 4)        # 4 K steps only
        assert lib.gemm_debug_force_tile(1, 6) == lib.STATUS_SUCCESS
        assert pick(1, 4096, 4096, 4096) == (6, 1)     # direct-to-LDS tiles never split
        assert lib.gemm_debug_force_tile(1, 0) == lib.STATUS_SUCCESS
        assert lib.gemm_debug_force_splits(1, 32) == lib.STATUS_SUCCESS
        assert pick(1, 4096, 4096, 4096) == (0, 1)     # 32 x 64 MiB exceeds the workspace
        assert pick(1, 1024, 1024, 8192) == (0, 16)    # 16 M floats: 16 partials fit
    finally:
        lib.gemm_debug_force_tile(1, -1)
        lib.gemm_debug_force_splits(1, -1)


def test_half_tile_resolution(so):
    """A forced direct-to-LDS tile takes any M, N, K with N a multiple of 8 (ragged
    edges and K run its bounds-checked instantiation); otherwise it is reported (and
    run) as the register-staged 256x256 configuration."""
    try:
        assert lib.gemm_debug_force_tile(1, 3) == lib.STATUS_SUCCESS
        assert pick(1, 4096, 4096, 4096)[0] == 3
        assert pick(1, 300, 512, 4096)[0] == 3
        assert pick(1, 512, 512, 96)[0] == 3
        assert pick(1, 512, 516, 96)[0] == 0       # N not a multiple of 8, packing not worth it
        assert pick(1, 1024, 1028, 1024)[0] == 3   # N not a multiple of 8: B packed
        assert lib.gemm_debug_force_tile(1, 4) == lib.STATUS_SUCCESS
        assert pick(1, 128, 256, 64)[0] == 4
        assert pick(1, 128, 128, 64)[0] == 4
        assert pick(1, 128, 132, 64)[0] == 0
        assert lib.gemm_debug_force_tile(1, 1) == lib.STATUS_SUCCESS
        assert pick(1, 128, 128, 64)[0] == 1
        # tile 7 splits the columns only where whole rounds plus one short round exist
        assert lib.gemm_debug_force_tile(1, 7) == lib.STATUS_SUCCESS
        assert pick(1, 4096, 14336, 4096)[0] == 7    # 768 + 256 half tiles
        assert pick(1, 4096, 4096, 4096)[0] == 6     # 256 tiles: whole rounds already
        assert pick(1, 4096, 5120, 128)[0] == 7
        assert pick(1, 4096, 5120, 128, cus=128)[0] == 7   # 2 rounds + 128 half tiles
        assert pick(1, 4096, 5120, 128, cus=64)[0] == 6    # the tail would need 2 rounds
        assert pick(1, 300, 5120, 128)[0] == 6     # ragged M: no split, the eight-wave tile
        assert pick(1, 300, 5124, 128)[0] == 6     # N not a multiple of 8: B packed
        assert pick(1, 64, 5124, 32)[0] == 0       # packing costs more than it saves
    finally:
        lib.gemm_debug_force_tile(1, -1)


def test_config_tuned_entries_are_used(so):
    """Every tuned entry is what the library runs for a shape of that size class
    (before the legality clamps, which cannot bind at these aligned sizes)."""
    for line in open(TUNED_TABLE):
        m = re.match(r"\s*\{\s*(-?\d+)\s*,\s*(\d+)\s*,\s*(\d+)\s*,\s*(\d+)\s*,"
                     r"\s*(\d+)\s*,\s*(\d+)\s*\}", line)
        if not m:
            continue
        op, lm, ln, lk, tile, splits = (int(g) for g in m.groups())
        M, N, K = 1 << lm, 1 << ln, 1 << lk
        got = pick(op, M, N, K)
        if op == 0 and splits > 1 and K <= 2048 and -(-M // 16) * -(-N // 16) <= 256:
            # small outputs that would split K across workgroups take the 16x16 tile,
            # whose waves split K inside the workgroup
            assert got == (13, 1), (op, M, N, K, got)
            continue
        # tile 7 of the half products runs as 6 where the shape has no head/tail split
        assert got[0] == tile or (op, tile, got[0]) == (1, 7, 6), (op, M, N, K, got, tile)
        if op == 0 and splits * M * N <= (64 << 20) // 4 and splits <= -(-K // 32):
            assert got[1] == splits, (op, M, N, K, got, splits)


def bk_of(tile):
    return 64 if tile == 13 else 32 if tile == 3 or tile >= 7 else 16


def test_split_legality(so):
    """Forced split counts are reduced to what K and the 64 MiB workspace allow,
    with no empty K chunk."""
    rng = random.Random(7)
    try:
        for _ in range(400):
            M, N = rng.randint(1, 3000), rng.randint(1, 3000)
            K = rng.choice([1, 15, 16, 17, 100, 777, 4096, 20000])
            want = rng.choice([1, 2, 3, 5, 8, 16, 32])
            tile = rng.choice([-1, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12])
            assert lib.gemm_debug_force_tile(0, tile) == lib.STATUS_SUCCESS
            assert lib.gemm_debug_force_splits(0, want) == lib.STATUS_SUCCESS
            t, s = pick(0, M, N, K)
            if tile >= 0:
                # direct-to-LDS tiles (7-11) run as their register-staged twin (4, or 2
                # for 11) where the operands do not allow copies (N % 4 != 0 and no packing)
                assert t == tile or (tile, t) in ((7, 4), (8, 4), (9, 4), (10, 4), (11, 2))
                if t != tile:
                    assert N % 4 != 0 or K % 4 != 0
            # the chunks are planned in the K granularity of the tile asked for (the
            # tuned or forced one) before a direct-to-LDS tile resolves to tile 4
            ok = False
            for bk in {bk_of(t), 32}:
                ktiles = -(-K // bk)
                if not 1 <= s <= max(1, min(want, ktiles)):
                    continue
                if s > 1:
                    chunk = -(-ktiles // min(want, ktiles, (64 << 20) // 4 // (M * N))) * bk
                    if not (s == -(-K // chunk) and (s - 1) * chunk < K):
                        continue
                ok = True
            assert ok, (M, N, K, want, tile, t, s)
            assert s * M * N <= (64 << 20) // 4 or s == 1
    finally:
        lib.gemm_debug_force_tile(0, -1)
        lib.gemm_debug_force_splits(0, -1)


def test_forced_splits(so):
    try:
        assert lib.gemm_debug_force_tile(0, 2) == lib.STATUS_SUCCESS
        assert lib.gemm_debug_force_splits(0, 8) == lib.STATUS_SUCCESS
        assert pick(0, 256, 256, 256) == (2, 8)        # 16 K tiles, 2 per chunk
        assert pick(0, 256, 256, 100) == (2, 7)        # only 7 K tiles
        assert pick(0, 8192, 8192, 8192) == (2, 1)     # 8 x 256 MiB exceeds the workspace
        assert pick(0, 2048, 2048, 4096) == (2, 4)     # 4 x 16 MiB fits exactly
        assert lib.gemm_debug_force_splits(0, 3) == lib.STATUS_SUCCESS
        assert pick(0, 64, 64, 160) == (2, 3)          # 10 K tiles -> chunks of 4, 4, 2
        assert lib.gemm_debug_force_splits(0, 1) == lib.STATUS_SUCCESS
        assert pick(0, 64, 64, 16384) == (2, 1)
    finally:
        lib.gemm_debug_force_tile(0, -1)
        lib.gemm_debug_force_splits(0, -1)
    assert lib.gemm_debug_force_splits(0, 0) == lib.STATUS_INVALID_VALUE
    assert lib.gemm_debug_force_splits(0, 33) == lib.STATUS_INVALID_VALUE
    assert lib.gemm_debug_force_splits(2, 2) == lib.STATUS_INVALID_VALUE
    assert lib.gemm_debug_force_splits(1, 33) == lib.STATUS_INVALID_VALUE
    assert lib.gemm_debug_force_splits(0, -1) == lib.STATUS_SUCCESS
    with pytest.raises(lib.GemmError):
        pick(2, 300, 500, 64)
    with pytest.raises(lib.GemmError):
        pick(0, -1, 500, 64)
    with pytest.raises(lib.GemmError):
        pick(0, 300, 500, 64, cus=0)


def test_force_tile_values(so):
    assert lib.gemm_debug_force_tile(0, 14) == lib.STATUS_INVALID_VALUE
    assert lib.gemm_debug_force_tile(0, 13) == lib.STATUS_SUCCESS
    assert lib.gemm_debug_force_tile(0, 12) == lib.STATUS_SUCCESS
    assert lib.gemm_debug_force_tile(0, 11) == lib.STATUS_SUCCESS
    assert lib.gemm_debug_force_tile(0, 9) == lib.STATUS_SUCCESS
    assert lib.gemm_debug_force_tile(1, 10) == lib.STATUS_INVALID_VALUE
    assert lib.gemm_debug_force_tile(1, 9) == lib.STATUS_SUCCESS
    assert lib.gemm_debug_force_tile(1, 8) == lib.STATUS_SUCCESS
    assert lib.gemm_debug_force_tile(1, 7) == lib.STATUS_SUCCESS
    assert lib.gemm_debug_force_tile(1, 5) == lib.STATUS_SUCCESS
    assert lib.gemm_debug_force_tile(1, 3) == lib.STATUS_SUCCESS
    assert lib.gemm_debug_force_tile(1, -1) == lib.STATUS_SUCCESS
    assert lib.gemm_debug_force_tile(0, 4) == lib.STATUS_SUCCESS
    assert lib.gemm_debug_force_tile(5, 0) == lib.STATUS_INVALID_VALUE
    assert lib.gemm_debug_force_tile(0, -1) == lib.STATUS_SUCCESS


def test_tuner_covers_every_tile(so):
    """The tuner times (and names in its report) exactly the tile configurations the
    library accepts."""
    from linear_algebra_sgemm_amd import tune
    try:
        for op, tiles in ((0, tune.SGEMM_TILES), (1, tune.HALF_TILES)):
            valid = {t for t in range(32) if lib.gemm_debug_force_tile(op, t) == lib.STATUS_SUCCESS}
            assert valid == set(tiles) == set(tune.TILE_NAMES[op]), (op, valid, tiles)
    finally:
        lib.gemm_debug_force_tile(0, -1)
        lib.gemm_debug_force_tile(1, -1)
