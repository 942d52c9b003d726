"""A seeded sweep of small whole-step shapes through the HIP path against the oracle:
each case draws the KV format, the index-key format, the KV-head count (1, 2, 3, 4 or
8), k, n_init / n_local, the context lengths (some short enough for -1 padding, some
ending on a page boundary), the verify length, the split count, one selection per row
or per KV head, and the launch mode (fused with the selection in the decode or in the
scoring launch, or the five separate calls). The bars are those of the other parity
tests (scores, selection validity and exactness where the gap qualifies, outputs on
the GPU's own selection)."""
import numpy as np
import pytest

from synth import workloads as W
from tests import gpu_common as G

pytestmark = pytest.mark.gpu

N_CASES = 64


def _case(i):
    r = np.random.default_rng([2026, i])
    hkv = int(r.choice([1, 2, 3, 4, 8]))
    k = int(r.choice([1, 2, 3, 5, 8, 16, 24, 64]))
    n_init = int(r.integers(0, 3)) if k >= 4 else 0
    n_local = int(r.integers(1, 3)) if k - n_init >= 2 else 1
    n_append = int(r.choice([0, 1, 2, 4]))
    B = int(r.integers(1, 5))
    lens = []
    for _ in range(B):
        kind = r.integers(0, 4)
        if kind == 0:
            L = int(r.integers(1, 400))                    # few blocks: -1 padding
        elif kind == 1:
            L = 128 * int(r.integers(1, 40)) - n_append   # the last row ends a page
        else:
            L = int(r.integers(400, 9000))
        lens.append(max(L, 1))
    splits = int(r.choice([s for s in (1, 2, 3, 4, 8, 16) if s <= k]))
    mode = str(r.choice(["fused", "fused", "score", "separate"]))
    if mode == "fused" and splits > 16:
        splits = 16
    tables = hkv if (hkv in (2, 4) and r.random() < 0.3) else 1   # (4 index heads split evenly)
    return dict(fmt=int(r.choice([W.FMT_FP8, W.FMT_NVFP4])),
                index_fmt=int(r.choice([W.IDX_E4M3, W.IDX_NVFP4])), hkv=hkv, k=k, n_init=n_init,
                n_local=n_local, n_append=n_append, lens=lens, splits=splits, mode=mode, tables=tables,
                seed=3000 + i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_small_step(M, i):
    c = _case(i)
    print("random step", i, c, flush=True)
    wl = W.small(c["fmt"], c["lens"], c["n_append"], num_kv_heads=c["hkv"], k=c["k"], seed=c["seed"],
                 index_fmt=c["index_fmt"])
    wl.n_init, wl.n_local = c["n_init"], c["n_local"]
    fused = c["mode"] != "separate"
    select_in = "score" if c["mode"] == "score" else "decode"
    G.check_step_parity(M, wl, c["splits"], fused, tables=c["tables"], select_in=select_in)


@pytest.fixture(scope="module")
def M():
    import sparse_attention_decode_fp8_amd as M
    return M
