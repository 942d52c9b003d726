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


N_UNION_CASES = 24


def _union_case(i):
    r = np.random.default_rng([2027, i])
    hkv = int(r.choice([1, 2, 4, 8]))
    k = int(r.choice([1, 3, 5, 8, 16, 32]))
    n_append = int(r.choice([2, 3, 4]))
    lens = [max(1, int(x)) for x in r.integers(1, 7000, size=int(r.integers(1, 4)))]
    return dict(fmt=int(r.choice([W.FMT_FP8, W.FMT_NVFP4])), hkv=hkv, k=k, n_append=n_append, lens=lens,
                overlap=float(r.choice([0.0, 0.5, 0.9, 1.0])), group=int(r.integers(1, 5)),
                splits=int(r.choice([1, 2, 3, 5, 9])), pages=bool(r.random() < 0.5),
                tables=hkv if (hkv in (2, 4) and r.random() < 0.3) else 1, seed=4000 + i)


@pytest.mark.parametrize("i", range(N_UNION_CASES))
def test_random_union_decode(M, i):
    import torch
    from oracle import msa_oracle as O
    c = _union_case(i)
    print("random union", i, c, flush=True)
    wl = W.small(c["fmt"], c["lens"], c["n_append"], num_kv_heads=c["hkv"], k=c["k"], seed=c["seed"])
    pool = G.gpu_pool(M, wl)
    sl, kb, vb, ib = wl.step_tokens()
    M.msa_kv_append(pool, torch.from_numpy(sl).cuda(), G.dev_bf16(kb), G.dev_bf16(vb), G.dev_bf16(ib))
    if c["tables"] > 1:
        sel = np.stack([W.verify_tables(wl, c["overlap"], seed_tag=5 + t) for t in range(c["tables"])], axis=1)
    else:
        sel = W.verify_tables(wl, c["overlap"])
    pages = None
    if c["pages"]:
        pages = np.where(sel >= 0, wl.block_table[wl.row_seq.reshape((-1,) + (1,) * (sel.ndim - 1)),
                                                  np.maximum(sel, 0)], -1).astype(np.int32)
    groups = M.group_rows_of(wl.row_seq, c["group"])
    step = M.Step(wl.block_table, wl.row_seq, wl.row_pos, sel_tables=c["tables"])
    q = G.dev_bf16(wl.q)
    sel_d = torch.from_numpy(np.ascontiguousarray(sel, dtype=np.int32)).cuda()
    pg_d = None if pages is None else torch.from_numpy(np.ascontiguousarray(pages)).cuda()
    gr = torch.from_numpy(groups).cuda()
    out = torch.zeros(wl.num_rows, wl.num_heads, 128, dtype=torch.bfloat16, device="cuda")
    ns = c["splits"]
    if ns == 1:
        M.msa_sparse_decode_union(pool, step, q, sel_d, wl.k, gr, c["group"], wl.softmax_scale, 1, out=out,
                                  sel_pages=pg_d)
    else:
        po = torch.zeros(wl.num_rows, wl.num_heads, ns, 128, device="cuda")
        pm = torch.zeros(wl.num_rows, wl.num_heads, ns, 2, device="cuda")
        M.msa_sparse_decode_union(pool, step, q, sel_d, wl.k, gr, c["group"], wl.softmax_scale, ns, part_o=po,
                                  part_ml=pm, sel_pages=pg_d)
        M.msa_combine(wl.num_rows, wl.num_heads, 128, ns, po, pm, out)
    torch.cuda.synchronize()
    opool = G.oracle_pool(wl)
    ref = O.attend(opool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel, wl.softmax_scale)
    G.assert_out_close(G.bf16_to_np(out), ref, f"union case {i}")
