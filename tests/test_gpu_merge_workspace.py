"""The fused entries' split-merge workspace: the fill entry sets the idle state, and one
workspace serves successive fused calls with different split counts, each equal bit
for bit to the separate decode + combine calls and each leaving the workspace idle."""
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


def test_workspace_init_sets_idle_state(M):
    rows, hq, S = 3, 32, 5
    po = torch.full((rows, hq, S, 128), 1.5, dtype=torch.float32, device="cuda")
    pm = torch.full((rows, hq, S, 2), -2.0, dtype=torch.float32, device="cuda")
    cnt = torch.full((rows, hq // 16), 9, dtype=torch.int32, device="cuda")
    guard = torch.full((64,), 3.0, dtype=torch.float32, device="cuda")
    M.msa_merge_workspace_init(rows, hq, 128, S, po, pm, cnt)
    torch.cuda.synchronize()
    assert bool((po.view(torch.int32) == M.MERGE_IDLE_BITS).all())
    assert bool((pm.view(torch.int32) == M.MERGE_IDLE_BITS).all())
    assert bool((cnt == 0).all())
    assert bool((guard == 3.0).all())


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_NVFP4])
def test_one_workspace_many_split_counts(M, fmt):
    wl = W.small(fmt, [3000, 700, 5000, 9000], 2, num_kv_heads=2, k=16, seed=81)
    print("merge workspace reuse", wl.name, flush=True)
    pool = G.gpu_pool(M, wl)
    step, q, q_idx, w, app = G.gpu_step_inputs(M, wl)
    kw = dict(slot=app[0], k_new=app[1], v_new=app[2], idx_k_new=app[3])
    big = M.DecodeBuffers(wl.num_rows, wl.num_heads, wl.max_blocks, wl.k, 16)
    M.msa_append_score_select(pool, step, q_idx, w, wl.k, wl.n_init, wl.n_local, big.block_scores, **kw)
    for ns in (8, 2, 16, 1, 3, 16, 5):
        print("  splits", ns, flush=True)
        ref = M.DecodeBuffers(wl.num_rows, wl.num_heads, wl.max_blocks, wl.k, ns)
        M.msa_select_topk(step, big.block_scores, wl.k, wl.n_init, wl.n_local, ref.sel, ref.sel_pages)
        M.msa_sparse_decode(pool, step, q, ref.sel, wl.k, wl.softmax_scale, ns, ref.part_o, ref.part_ml,
                            sel_pages=ref.sel_pages)
        M.msa_combine(wl.num_rows, wl.num_heads, 128, ns, ref.part_o, ref.part_ml, ref.out)
        big.out.fill_(0)
        M.msa_select_decode_combine(pool, step, q, big.block_scores, wl.k, wl.n_init, wl.n_local,
                                    wl.softmax_scale, ns, big.merge_o, big.merge_ml, big.counters,
                                    big.out, sel=big.sel, sel_pages=big.sel_pages)
        torch.cuda.synchronize()
        assert torch.equal(big.sel, ref.sel)
        assert torch.equal(big.out.view(torch.int16), ref.out.view(torch.int16)), ns
        G.assert_merge_idle(big)
        # the table-driven combining entry on the same workspace
        big.out.fill_(0)
        M.msa_sparse_decode_combine(pool, step, q, ref.sel, wl.k, wl.softmax_scale, ns, big.merge_o,
                                    big.merge_ml, big.counters, big.out, sel_pages=ref.sel_pages)
        torch.cuda.synchronize()
        assert torch.equal(big.out.view(torch.int16), ref.out.view(torch.int16)), ns
        G.assert_merge_idle(big)
    assert np.isfinite(G.bf16_to_np(big.out)).all()
