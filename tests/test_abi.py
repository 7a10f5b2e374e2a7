"""The C-ABI library loads, exports every entry point include/pka.h declares,
and rejects bad arguments on the host before launching anything.  CPU only:
no call here reaches a GPU (every call fails validation first or is a pure
host function)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pka.h")


def _declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pka_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def pka():
    import paged_kv_attention_21_amd as pka

    return pka


def test_header_declares_the_boundary():
    syms = _declared_symbols()
    for name in ("pka_kv_cache_write", "pka_paged_attn_decode", "pka_paged_attn_decode_v1",
                 "pka_paged_attn_decode_splitk", "pka_paged_attn_splitk_reduce", "pka_paged_attn_prefill",
                 "pka_splitk_workspace_bytes", "pka_decode_choose_variant", "pka_status_str",
                 "pka_prefill_workspace_bytes", "pka_prefill_split_keys", "pka_rope_table", "pka_rope_table_bytes", "pka_fused_rope_kv_write",
                 "pka_paged_attn_decode_append"):
        assert name in syms


def test_library_exports_every_declared_symbol(pka):
    lib = ctypes.CDLL(pka.LIB_PATH)
    missing = [s for s in _declared_symbols() if not hasattr(lib, s)]
    assert not missing, f"declared but not exported: {missing}"


def test_status_strings_and_version(pka):
    lib = pka._lib.lib
    for code in range(7):
        assert lib.pka_status_str(code).decode()
    assert lib.pka_status_str(99).decode() == "unknown status"
    assert pka.version() >= 100


def _desc(pka, nb=64, bs=16, hkv=2, d=64, dt=0):
    return pka.CacheDesc(nb, bs, hkv, d, dt)


A = 4096  # a 16-byte aligned fake address: never dereferenced, every call below fails validation first


def test_kv_write_validation(pka):
    lib = pka._lib.lib
    d = _desc(pka)
    assert lib.pka_kv_cache_write(A, A, A, -1, A, A, d, None) == 2
    assert lib.pka_kv_cache_write(A, A, A, 0, A, A, d, None) == 0  # empty: no-op
    assert lib.pka_kv_cache_write(None, A, A, 4, A, A, d, None) == 1
    assert lib.pka_kv_cache_write(A + 2, A, A, 4, A, A, d, None) == 4
    assert lib.pka_kv_cache_write(A, A, A, 4, A, A, _desc(pka, bs=64), None) == 3
    assert lib.pka_kv_cache_write(A, A, A, 4, A, A, _desc(pka, d=96), None) == 3
    assert lib.pka_kv_cache_write(A, A, A, 4, A, A, _desc(pka, dt=7), None) == 3
    assert lib.pka_kv_cache_write(A, A, A, 4, A, A, _desc(pka, nb=0), None) == 2


def test_decode_validation(pka):
    lib = pka._lib.lib
    d = _desc(pka)
    v1 = lib.pka_paged_attn_decode_v1
    assert v1(A, A, A, A, A, 0, 2, 8, 0.125, A, d, None) == 0      # no sequences: no-op
    assert v1(A, A, A, A, A, -1, 2, 8, 0.125, A, d, None) == 2
    assert v1(None, A, A, A, A, 1, 2, 8, 0.125, A, d, None) == 1
    assert v1(A, A, A, A, A, 1, 2, 8, 0.125, None, d, None) == 1
    assert v1(A, A, A, A, A, 1, 3, 8, 0.125, A, d, None) == 2       # Hq % Hkv
    assert v1(A, A, A, A, A, 1, 6, 8, 0.125, A, d, None) == 3       # group 3 not built
    assert v1(A, A, A, A, A, 1, 2, 0, 0.125, A, d, None) == 2
    assert v1(A + 8, A, A, A, A, 1, 2, 8, 0.125, A, d, None) == 4
    assert v1(A, A, A, A, A, 1, 2, 8, 0.125, A + 4, d, None) == 4
    sk = lib.pka_paged_attn_decode_splitk
    assert sk(A, A, A, A, A, 1, 2, 8, 0.125, 128, 4, A, A, A, d, None) == 3  # partition size must be 256
    assert sk(A, A, A, A, A, 1, 2, 8, 0.125, 256, 4, None, A, A, d, None) == 5
    assert sk(A, A, A, A, A, 1, 2, 8, 0.125, 256, 0, A, A, A, d, None) == 2
    red = lib.pka_paged_attn_splitk_reduce
    assert red(A, A, A, A, 1, 2, 96, 256, 4, A, 0, None) == 3
    assert red(A, A, A, A, 1, 2, 64, 256, 4, None, 0, None) == 1
    assert red(A, A, A, A, 0, 2, 64, 256, 4, A, 0, None) == 0
    auto = lib.pka_paged_attn_decode
    assert auto(A, A, A, A, A, 1, 2, 8, 0, 0.125, A, d, None, 0, None) == 2  # max_context_len 0
    assert auto(A, A, A, None, A, 1, 2, 8, 128, 0.125, A, d, None, 0, None) == 1
    app = lib.pka_paged_attn_decode_append
    assert app(A, A, A, A, A, A, A, 0, 2, 8, 128, 0.125, A, d, None, 0, None) == 0      # no sequences: no-op
    assert app(A, None, A, A, A, A, A, 1, 2, 8, 128, 0.125, A, d, None, 0, None) == 1   # no new K rows
    assert app(A, A, None, A, A, A, A, 1, 2, 8, 128, 0.125, A, d, None, 0, None) == 1   # no new V rows
    assert app(A, A + 2, A, A, A, A, A, 1, 2, 8, 128, 0.125, A, d, None, 0, None) == 4  # misaligned rows
    assert app(A, A, A, A, A, None, A, 1, 2, 8, 128, 0.125, A, d, None, 0, None) == 1   # no block tables
    assert app(A, A, A, A, A, A, A, 1, 2, 8, 0, 0.125, A, d, None, 0, None) == 2        # max_context_len 0


def test_prefill_validation(pka):
    lib = pka._lib.lib
    d = _desc(pka, hkv=8, d=128, dt=1)
    pf = lib.pka_paged_attn_prefill
    assert pf(A, A, A, A, A, A, 0, 0, 0, 0, 16, 8, 0.1, A, d, None, 0, None) == 0
    assert pf(A, A, A, A, A, None, 2, 10, 5, 100, 16, 8, 0.1, A, d, None, 0, None) == 1
    assert pf(A, A, A, A, A, A, 2, 10, 11, 100, 16, 8, 0.1, A, d, None, 0, None) == 2  # max_query_len > num_q_tokens
    assert pf(A, A, A, A, A, A, 2, 10, 5, 4, 16, 8, 0.1, A, d, None, 0, None) == 2     # max_context_len < max_query_len
    assert pf(A, A, A, A, A, A, 2, 10, 5, 100, 12, 8, 0.1, A, d, None, 0, None) == 2   # 12 % 8
    bad = _desc(pka, bs=64, hkv=8, d=128, dt=1)
    assert pf(A, A, A, A, A, A, 2, 10, 5, 100, 128, 8, 0.1, A, d, None, 0, None) == 3    # GQA group 16
    assert pf(A, A, A, A, A, A, 2, 10, 5, 100, 16, 8, 0.1, A, bad, None, 0, None) == 3
    for scale in (0.0, -0.1, float("inf"), float("nan")):  # the running max assumes a positive scale
        assert pf(A, A, A, A, A, A, 2, 10, 5, 100, 16, 8, scale, A, d, None, 0, None) == 3
    # a tile can see more keys than one split holds: the workspace is required
    assert pf(A, A, A, A, A, A, 2, 10, 5, 5000, 16, 8, 0.1, A, d, None, 0, None) == 5
    need = pka.prefill_workspace_bytes(2, 10, 16, 8, 128, 5000)
    assert need > 0
    # no split when every query tile fits in one split: a context no longer
    # than the shortest split, or enough query tiles to fill the GPU
    assert pka.prefill_workspace_bytes(2, 10, 16, 8, 128, 256) == 0
    assert pka.prefill_workspace_bytes(4, 8192, 16, 8, 128, 8192) == 0


def _prefill_splits(num_seqs, num_q_tokens, hkv, group, max_ctx, d=128, cus=256):
    """The split count the library's policy gives (restated from its
    definition: about four (query tile, KV head) items per compute unit - two
    at head size 256, whose workgroups take a whole compute unit -, splits of
    at least 256 keys and, in batches where that keeps the items within twice
    the target, of at most 1,024; whole 64-key tiles)."""
    tiles = -(-num_q_tokens // (128 // group)) + num_seqs
    items = tiles * hkv
    target = (2 if d > 128 else 4) * cus
    s = 1 if items >= target else -(-target // items)
    s = min(s, max(1, -(-max_ctx // 256)))
    keys = -(-max_ctx // s)
    if s > 1 and keys > 1024 and items * -(-max_ctx // 1024) <= 2 * target:
        keys = 1024
    keys = max(64, -(-keys // 64) * 64)
    return -(-max_ctx // keys), tiles


@pytest.mark.parametrize("shape", [(2, 10, 8, 2, 5000, 128), (5, 1984, 8, 2, 3072, 128), (5, 1984, 8, 2, 5632, 128),
                                   (4, 2048, 8, 2, 16896, 128),
                                   (1, 7, 2, 1, 4096, 128), (8, 4096, 8, 2, 8192, 128), (3, 300, 4, 4, 700, 128),
                                   (4, 8192, 4, 2, 8192, 256), (4, 8192, 4, 2, 8192, 128), (2, 600, 4, 2, 3000, 256),
                                   (3, 300, 4, 4, 700, 64)])
def test_prefill_split_policy(pka, shape):
    """The workspace the library asks for is the split states of exactly the
    split count the policy gives (CPU: the 256-CU default).  The long prefill
    at head size 256 with 4 KV heads fills two rounds of one workgroup per
    compute unit unsplit; at 128 dims the same batch is split in two."""
    ns, nq, hkv, g, ctx, d = shape
    splits, tiles = _prefill_splits(ns, nq, hkv, g, ctx, d)
    want = 0 if splits <= 1 else tiles * splits * hkv * 128 * (d + 2) * 4
    assert pka.prefill_workspace_bytes(ns, nq, hkv * g, hkv, d, ctx) == want
    keys = pka.prefill_split_keys(ns, nq, hkv * g, hkv, d, ctx)
    assert keys % 64 == 0 and -(-ctx // keys) == splits


def test_workspace_bytes_and_dispatcher(pka):
    # config-4 shape: the 64 KiB header of arrival counters, then 4 seqs x 16 heads
    # x 64 partitions x 128 dims fp32, plus max/sum arrays
    rows = 4 * 16 * 64
    assert pka.splitk_workspace_bytes(4, 16, 128, 16384) == (65536 + rows * 128 * 4
                                                             + 2 * ((rows * 4 + 255) // 256 * 256))
    assert pka.splitk_workspace_bytes(0, 16, 128, 100) == 0
    cv = pka.decode_choose_variant
    assert cv(1, 2, 128, 256) == 1            # one partition: nothing to split
    assert cv(1, 2, 4096, 256) == 2           # single long request
    assert cv(4, 8, 16384, 256) == 2          # few sequences, long contexts
    assert cv(256, 8, 2048, 256) == 1         # 2048 (seq, head) workgroups on 256 CUs
    assert cv(64, 8, 2048, 256) == 1          # mixed-step decodes: 512 workgroups, contexts <= 2048
    assert cv(32, 8, 2048, 256) == 2          # 256 workgroups: one per CU, split instead
    assert cv(64, 8, 8192, 256) == 2          # long contexts: split


def test_rope_validation(pka):
    """Host-side checks of the RoPE entry points (nothing is launched)."""
    lib = pka._lib.lib
    d = _desc(pka, hkv=8, d=128, dt=1)
    assert lib.pka_rope_table_bytes(4096, 128) == 4096 * 128 * 4
    assert lib.pka_rope_table_bytes(0, 128) == 0
    assert lib.pka_rope_table(A, 10, 100, 1e4, None) == 2       # head_dim not a multiple of 16
    assert lib.pka_rope_table(A, 10, 128, 1.0, None) == 2       # theta must exceed 1
    assert lib.pka_rope_table(None, 10, 128, 1e4, None) == 1
    assert lib.pka_rope_table(A, 0, 128, 1e4, None) == 0        # nothing to fill
    f = lib.pka_fused_rope_kv_write
    row = (16 + 16) * 128
    assert f(A, row, A, A, 0, 16, A, 4096, A, A, A, d, None) == 0          # no tokens
    assert f(A, row - 8, A, A, 4, 16, A, 4096, A, A, A, d, None) == 2      # stride below the row
    assert f(A, row + 4, A, A, 4, 16, A, 4096, A, A, A, d, None) == 2      # rows not 16-byte aligned
    assert f(A, row, None, A, 4, 16, A, 4096, A, A, A, d, None) == 1
    assert f(A, row, A, A, 4, 16, A, 0, A, A, A, d, None) == 2             # empty table
    assert f(A, row, A, A, 4, 0, A, 4096, A, A, A, d, None) == 2           # no q heads
