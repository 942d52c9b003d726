"""Parity of the whole decode step at the five benchmark workloads' full sizes, in
the launch configuration the benchmark times. Block scores, selection tables and
outputs are checked on sampled query rows that the oracle computes one by one; the
appended tokens' page bytes are checked exactly."""
import numpy as np
import pytest
import torch

from oracle import msa_oracle as O
from sparse_attention_decode_fp8_amd.pipeline import default_num_splits
from synth import workloads as W
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


def _sample_rows(wl, cfg, n=8):
    rows = wl.num_rows
    if rows <= n:
        return list(range(rows))
    rng = np.random.default_rng(cfg)
    pick = set(rng.choice(rows, size=n, replace=False).tolist())
    nb = wl.row_pos // 128 + 1
    pick |= set(np.nonzero(nb <= wl.k)[0][:3].tolist())          # dense rows, if any
    pick.add(int(np.argmax(wl.row_pos)))                          # the longest row
    return sorted(pick)


@pytest.mark.parametrize("cfg,index_fmt", [(0, W.IDX_E4M3), (1, W.IDX_E4M3), (2, W.IDX_E4M3),
                                           (3, W.IDX_E4M3), (4, W.IDX_E4M3), (1, W.IDX_NVFP4)])
def test_config_parity(cfg, index_fmt):
    import sparse_attention_decode_fp8_amd as M
    wl = W.config(cfg, index_fmt=index_fmt)
    ns = default_num_splits(wl.k, wl.num_rows * wl.num_kv_heads)
    print(f"config {cfg} {wl.name}: rows {wl.num_rows} pages {wl.num_pages} splits {ns}", flush=True)
    pool = G.gpu_pool(M, wl)
    bufs = G.run_gpu_step(M, wl, pool, ns)
    S_gpu = bufs.block_scores.cpu().numpy()
    sel_gpu = bufs.sel.cpu().numpy()
    out_gpu = G.bf16_to_np(bufs.out)
    rows = _sample_rows(wl, cfg)
    S, sel, out, opool = G.oracle_rows(wl, rows)
    nb = wl.row_pos // 128 + 1
    exact = 0
    for i, r in enumerate(rows):
        G.assert_scores_close(S_gpu[r:r + 1], S[i:i + 1])
        if G.gap_qualified(S[i], nb[r], wl.k, wl.n_init, wl.n_local):
            assert np.array_equal(sel_gpu[r], sel[i]), f"row {r}"
        else:
            G.check_selection_valid(sel_gpu[r], S[i], nb[r], wl.k, wl.n_init, wl.n_local)
        if np.array_equal(sel_gpu[r], sel[i]):
            exact += 1
            G.assert_out_close(out_gpu[r], out[i], f"row {r}")
    assert exact >= len(rows) - 1
    if cfg == 3:   # every row's selection is decided by the 1100-way tie: all exact
        assert exact == len(rows)
        for i, r in enumerate(rows):
            tied = wl.tie_blocks[int(wl.row_seq[r])]
            assert list(sel_gpu[r]) == sorted(list(tied[:wl.k - 1]) + [nb[r] - 1])
    # the step's appended tokens: page bytes exact for the sampled requests
    seqs = sorted(set(int(wl.row_seq[r]) for r in rows))
    arrays = {k: v.cpu().numpy() for k, v in pool.arrays().items()}
    for s in seqs:
        L = int(wl.ctx_lens[s])
        if wl.n_append == 0:
            continue
        pos = np.arange(L, L + wl.n_append)
        slots = wl.slots(s, pos)
        page, off = slots // 128, slots % 128
        O.kv_append(opool, slots, wl.k_src[s][pos], wl.v_src[s][pos], wl.idx_src[s][pos])
        names = ["k_codes", "v_codes", "index_k"]
        if wl.fmt == W.FMT_NVFP4:
            names += ["k_scales", "v_scales"]
        if wl.index_fmt == W.IDX_NVFP4:
            names += ["index_scales"]
        for name in names:
            g = arrays[name].reshape(opool[name].shape)
            if name.startswith("index") and wl.index_fmt == W.IDX_NVFP4:   # [page][g][n][t]
                assert np.array_equal(g[page, :, off % 16, off // 16],
                                      opool[name][page, :, off % 16, off // 16]), name
            elif name.startswith("index"):
                assert np.array_equal(g[page, off], opool[name][page, off])
            else:
                assert np.array_equal(g[page, :, off], opool[name][page, :, off]), name
    print(f"config {cfg}: {len(rows)} rows checked, {exact} selections identical", flush=True)
