"""Host-side logic without a GPU: the split-count policy and the benchmark's
algorithmic-byte count (union of a request's selected visible tokens per KV head)."""
import importlib.util
import os
import types

import numpy as np

from sparse_attention_decode_fp8_amd.pipeline import FUSED_APPEND_MAX, default_num_splits

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_default_num_splits_policy():
    # about 256 workgroups, a power of two, at most min(k, 16)
    assert default_num_splits(16, 32) == 8      # config 1: 8 rows x 4 KV heads
    assert default_num_splits(8, 1) == 8        # config 0: one block per split
    assert default_num_splits(32, 8) == 16      # config 3: capped at 16
    assert default_num_splits(16, 640) == 1     # config 2: the pairs fill the GPU
    assert default_num_splits(16, 192) == 1     # config 4
    assert default_num_splits(1, 1) == 1
    for k in range(1, 65):
        for pairs in (1, 3, 17, 100, 256, 1000):
            s = default_num_splits(k, pairs)
            assert s >= 1 and (s & (s - 1)) == 0 and s <= min(k, 16) and s * pairs <= max(256, pairs)
    assert FUSED_APPEND_MAX == 64


def test_algorithmic_bytes_count_the_union_per_request_and_kv_head():
    B = _bench()
    # two requests: request 0 has rows at positions 300 and 301 (3 blocks, the last
    # with 45 / 46 visible tokens), request 1 one row at position 127 (one full block)
    wl = types.SimpleNamespace(ctx_lens=np.array([300, 127]), row_seq=np.array([0, 0, 1]),
                               row_pos=np.array([300, 301, 127]), num_kv_heads=2, num_rows=3, num_heads=32)
    sel = np.array([[0, 2], [1, 2], [0, -1]], dtype=np.int32)
    total, tok = B.decode_algorithmic_bytes(wl, sel, 144)
    # request 0: blocks {0, 1, 2}: 128 + 128 + 46 (the later row sees token 301) = 302
    # request 1: block 0, 128 tokens
    assert tok == 302 + 128
    qo = 2 * 3 * 32 * 128 * 2
    meta = sel.size * 4 + 5 * 4
    assert total == (302 + 128) * 2 * 144 + qo + meta
    # per-KV-head tables: each KV head counts its own union
    sel3 = np.array([[[0, 2], [1, 2]], [[1, 2], [1, 2]], [[0, -1], [0, -1]]], dtype=np.int32)
    total3, tok3 = B.decode_algorithmic_bytes(wl, sel3, 144)
    head0 = 302 + 128                      # blocks {0,1,2} of request 0, block 0 of request 1
    head1 = (128 + 46) + 128               # blocks {1, 2} of request 0, block 0 of request 1
    assert total3 == (head0 + head1) * 144 + qo + sel3.size * 4 + int((sel3 >= 0).sum()) * 4
    assert tok3 == (head0 + head1) // 2


def test_read_floor_units_are_the_union_per_request_and_kv_head():
    B = _bench()
    wl = types.SimpleNamespace(ctx_lens=np.array([300, 127]), row_seq=np.array([0, 0, 1]),
                               row_pos=np.array([300, 301, 127]), num_kv_heads=2, num_rows=3, num_heads=32,
                               block_table=np.array([[7, 3, 9], [5, -1, -1]], dtype=np.int32))
    sel = np.array([[0, 2], [1, 2], [0, -1]], dtype=np.int32)
    u = B.selected_units(wl, sel)
    want = [(7, 0, 128), (3, 0, 128), (9, 0, 46), (7, 1, 128), (3, 1, 128), (9, 1, 46), (5, 0, 128), (5, 1, 128)]
    assert sorted(map(tuple, u.tolist())) == sorted(want)
    # the units hold exactly the tokens the algorithmic bytes count, per KV head
    total, tok = B.decode_algorithmic_bytes(wl, sel, 144)
    assert int(u[:, 2].sum()) == tok * 2
    sel3 = np.array([[[0, 2], [1, 2]], [[1, 2], [1, 2]], [[0, -1], [0, -1]]], dtype=np.int32)
    u3 = B.selected_units(wl, sel3)
    assert sorted(map(tuple, u3.tolist())) == sorted([(7, 0, 128), (3, 0, 128), (9, 0, 46), (3, 1, 128),
                                                      (9, 1, 46), (5, 0, 128), (5, 1, 128)])


def test_auto_replicas_put_512_mib_between_reuses():
    B = _bench()
    # 8 rows of 32769 tokens, k 16, 4 KV heads, NVFP4: 9.44 MB of decode reads per step
    wl = types.SimpleNamespace(fmt=2, k=16, num_kv_heads=4, row_pos=np.full(8, 32768))
    est = 8 * 16 * 128 * 4 * 144
    r = B.auto_replicas(wl, 169 << 20)
    assert r % 8 == 0 and (r - 1) * est >= 512 << 20 and r == 64
    assert B.auto_replicas(wl, 1 << 30) == 48            # 48 GiB budget
    wl0 = types.SimpleNamespace(fmt=1, k=8, num_kv_heads=1, row_pos=np.array([4095]))
    assert B.auto_replicas(wl0, 2 << 20) == 512          # capped


def test_group_rows_keep_a_requests_rows_together_up_to_the_group_size():
    from sparse_attention_decode_fp8_amd import group_rows_of
    rs = np.array([0, 0, 0, 0, 1, 2, 2, 3, 3, 3, 3, 3])
    assert group_rows_of(rs, 4).tolist() == [0, 4, 5, 7, 11, 12]
    assert group_rows_of(rs, 2).tolist() == [0, 2, 4, 5, 7, 9, 11, 12]
    assert group_rows_of(rs, 1).tolist() == list(range(13))
    assert group_rows_of(np.zeros(0, np.int32), 4).tolist() == [0]
    # config 2's layout: 40 requests x 4 rows -> 40 groups of 4
    assert group_rows_of(np.repeat(np.arange(40), 4), 4).tolist() == list(range(0, 161, 4))


def test_rows_per_seq_of():
    """The Python Step states rows_per_seq only when every request has the same number
    of consecutive rows."""
    from sparse_attention_decode_fp8_amd._lib import rows_per_seq_of
    assert rows_per_seq_of([0, 0, 0, 0, 1, 1, 1, 1], 2) == 4
    assert rows_per_seq_of([0, 1, 2], 3) == 1
    assert rows_per_seq_of([0, 0, 0, 1, 1, 1, 1, 1], 2) == 0     # 3 and 5 rows
    assert rows_per_seq_of([0, 1, 0, 1], 2) == 0                 # not request-major
    assert rows_per_seq_of([0, 0, 1, 1], 3) == 0                 # request 2 has no rows
    assert rows_per_seq_of([], 2) == 0
