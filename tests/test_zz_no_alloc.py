"""msa_sparse_decode_combine_noalloc (the split partials in the library's fixed per-GPU
array) against msa_sparse_decode_combine with a caller-allocated merge workspace: the
same bf16 output bit for bit, on several calls in a row whose inputs shrink (the
array keeps the previous call's partials), with one split and with several; a call
too large for the array is refused before any launch."""
import numpy as np
import pytest
import torch

from synth import workloads as W
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import sparse_attention_decode_fp8_amd as M
    return M


def _print(*a):
    print(*a, flush=True)


def _reference(M, wl, pool, step, q, sel, ns):
    bufs = M.DecodeBuffers(wl.num_rows, wl.num_heads, wl.max_blocks, wl.k, ns)
    M.msa_sparse_decode_combine(pool, step, q, sel, wl.k, wl.softmax_scale, ns, bufs.merge_o, bufs.merge_ml,
                                bufs.counters, bufs.out)
    torch.cuda.synchronize()
    return bufs.out.clone()


def test_no_alloc_matches_the_workspace_entry_on_shrinking_calls(M):
    full = W.small(W.FMT_NVFP4, [3000, 5200, 2600, 4100], 2, num_kv_heads=4, k=8, seed=61)
    pool = G.gpu_pool(M, full)
    sl, kb, vb, ib = full.step_tokens()
    M.msa_kv_append(pool, torch.from_numpy(sl).cuda(), G.dev_bf16(kb), G.dev_bf16(vb), G.dev_bf16(ib))
    # (rows kept, splits): 8 rows over 4 splits, then 3 rows over 2, then 3 rows over 1,
    # then 2 rows over 4 again
    for keep, ns in (([0, 1, 2, 3, 4, 5, 6, 7], 4), ([2, 3, 6], 2), ([2, 3, 6], 1), ([0, 5], 4)):
        wl = W.keep_rows(full, keep)
        _print("no-alloc decode, rows", keep, "splits", ns)
        step = M.Step(wl.block_table, wl.row_seq, wl.row_pos)
        q = G.dev_bf16(wl.q)
        sel = torch.from_numpy(W.verify_tables(wl, 0.5)).cuda()
        want = _reference(M, wl, pool, step, q, sel, ns)
        got = torch.full_like(want, float("nan"))
        M.msa_sparse_decode_combine_noalloc(pool, step, q, sel, wl.k, wl.softmax_scale, ns, got)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (keep, ns)


def test_no_alloc_refuses_a_call_larger_than_its_array(M):
    wl = W.small(W.FMT_NVFP4, [600], 1, num_kv_heads=4, k=4, seed=62)
    pool = G.gpu_pool(M, wl)
    # 600 rows x 64 heads x 4 splits x 130 fp32 = 80 MB of partials > 8 MiB
    rows = 600
    step = M.Step(wl.block_table, np.zeros(rows, np.int32), np.full(rows, 599, np.int32))
    q = torch.zeros(rows, 64, 128, dtype=torch.bfloat16, device="cuda")
    sel = torch.zeros(rows, 4, dtype=torch.int32, device="cuda")
    out = torch.zeros(rows, 64, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(M.MsaError, match="TOO_LARGE"):
        M.msa_sparse_decode_combine_noalloc(pool, step, q, sel, 4, wl.softmax_scale, 4, out)
    assert int(out.view(torch.int16).abs().sum().item()) == 0
