"""NVFP4 index keys on the GPU against the oracle: appended key bytes bit-exact, the
whole step (scores, selection, outputs) within the stated bars, and exact ties for
identical keys."""
import numpy as np
import pytest
import torch

from oracle import msa_oracle as O
from synth import workloads as W
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import sparse_attention_decode_fp8_amd as M
    return M


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_NVFP4])
def test_append_index_bytes_bit_exact(M, fmt):
    wl = W.small(fmt, [1000, 300, 129], 2, num_kv_heads=2, k=4, seed=71, index_fmt=W.IDX_NVFP4)
    print("nvfp4 index append", wl.name, flush=True)
    pool = G.gpu_pool(M, wl)
    step, q, q_idx, w, app = G.gpu_step_inputs(M, wl)
    M.msa_kv_append(pool, *app)
    torch.cuda.synchronize()
    ref = G.oracle_pool(wl)
    got = pool.arrays()
    for name in ("index_k", "index_scales"):
        assert np.array_equal(got[name].cpu().numpy().reshape(-1), ref[name].reshape(-1)), name


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_NVFP4])
@pytest.mark.parametrize("num_splits,fused", [(2, True), (2, False)])
def test_full_step_parity_nvfp4_index(M, fmt, num_splits, fused):
    wl = W.small(fmt, [1000, 2600, 130, 640], 3, num_kv_heads=2, k=5, seed=72, index_fmt=W.IDX_NVFP4)
    print("nvfp4 index step", wl.name, "splits", num_splits, "fused", fused, flush=True)
    G.check_step_parity(M, wl, num_splits, fused)


def test_identical_nvfp4_keys_tie_exactly(M):
    wl = W.small(W.FMT_FP8, [128 * 40], 0, num_kv_heads=1, k=8, seed=73, index_fmt=W.IDX_NVFP4)
    W.inject_ties(wl, 20)
    print("nvfp4 index ties", wl.name, flush=True)
    pool = G.gpu_pool(M, wl)
    step, q, q_idx, w, _ = G.gpu_step_inputs(M, wl)
    S = torch.empty((1, wl.max_blocks), dtype=torch.float32, device="cuda")
    M.msa_index_score(pool, step, q_idx, w, S)
    S = S.cpu().numpy()[0]
    tied = wl.tie_blocks[0]
    assert len(set(S[tied].tolist())) == 1
    others = np.setdiff1d(np.arange(wl.max_blocks), tied)
    assert S[tied[0]] > S[others].max()
    ref = O.index_score(G.oracle_pool(wl), wl.block_table, wl.row_seq, wl.row_pos, wl.q_idx, wl.w,
                        wl.max_blocks)
    G.assert_scores_close(S[None], ref)
