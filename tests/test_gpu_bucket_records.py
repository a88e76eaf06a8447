"""The selection's bucket records (lsa_select's optional output) and their use by the
bucket-major attention: each record set expands to exactly the row's tokens (flat and
tree search), the attention over them equals the attention over the rows bit for bit,
and records that do not match their row send the row to the list path."""

import numpy as np
import pytest
import torch

import sparse_attention_indexing_latent_amd as lsa
from synth import get_config, layer_inputs
from tests.parity import tol_for

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def layer():
    print("[rec] generating inputs", flush=True)
    cfg = get_config(2, T=32768, H_kv=2, H_q=10, n_topics=64)
    inp = layer_inputs(cfg, seed=5)
    G = {k: inp[k].to(DEV).contiguous() for k in ("K", "V", "W", "Q", "q_pos")}
    cache = lsa.build_buckets(G["K"], G["W"], n_q_heads=cfg.H_q, build_tree=True)
    torch.cuda.synchronize()
    return dict(cfg=cfg, G=G, cache=cache,
                members=cache.members()[0].cpu().numpy().astype(np.int64) & 0xFFFF,
                meta=cache.meta()[0].cpu().numpy().astype(np.int64))


def _select(layer, search, **kw):
    cfg, G = layer["cfg"], layer["G"]
    beam = 64 if search == "tree" else 0
    return lsa.select(G["Q"], layer["cache"], G["q_pos"], G["W"], cfg.k, cfg.n_sinks, cfg.window, search=search,
                      beam=beam, **kw)


def _expand(rec_rows, n, members, meta, g):
    """Tokens of n records (leaf, mask lo, mask hi, 0): key j of a bucket is token 4 members[j/4] + j%4."""
    toks = []
    for r in rec_rows[:n]:
        leaf = int(r[0]) & 0xFFFFFFFF
        mask = (int(r[1]) & 0xFFFFFFFF) | ((int(r[2]) & 0xFFFFFFFF) << 32)
        blk = leaf // 64
        m = int(meta[g, leaf])
        size, off = m & 0xFF, (m >> 8) & 0x3FF
        assert mask != 0 and mask >> (4 * size) == 0, (leaf, hex(mask), size)
        mem = members[g, blk, off:off + size]
        toks += [blk * 2048 + 4 * int(mem[j // 4]) + j % 4 for j in range(4 * size) if (mask >> j) & 1]
    return toks


@pytest.mark.parametrize("search,strategy", [("flat", "auto"), ("flat", "materialized"), ("tree", "auto")])
def test_records_expand_to_the_rows(layer, search, strategy):
    lr0, cnt0 = _select(layer, search, strategy=strategy)
    lr, cnt, (recs, rcnt) = _select(layer, search, strategy=strategy, bucket_records=True)
    torch.cuda.synchronize()
    assert torch.equal(lr, lr0) and torch.equal(cnt, cnt0)
    lr, cnt, recs, rcnt = lr[0].cpu().numpy(), cnt[0].cpu().numpy(), recs[0].cpu().numpy(), rcnt[0].cpu().numpy()
    have = rcnt >= 0
    full = cnt == layer["cfg"].k
    print(f"[rec] {search}: records for {have.mean():.3f} of the rows ({have[full].mean():.3f} of the full ones)",
          flush=True)
    assert have[full].mean() > 0.9
    assert np.all(rcnt <= 256)
    rng = np.random.default_rng(2)
    cand = np.argwhere(have)
    for i, g in cand[rng.choice(len(cand), size=min(400, len(cand)), replace=False)]:
        n = int(rcnt[i, g])
        leaves = (recs[i, g, :n, 0].astype(np.int64) & 0xFFFFFFFF)
        assert np.all(np.diff(leaves) > 0), (i, g)
        toks = _expand(recs[i, g], n, layer["members"], layer["meta"], g)
        row = lr[i, g, :int(cnt[i, g])]
        assert len(toks) == len(row) and np.array_equal(np.sort(toks), row), (search, i, g)


@pytest.mark.parametrize("search", ["flat", "tree"])
def test_attention_over_records_is_bit_identical(layer, search):
    cfg, G = layer["cfg"], layer["G"]
    lr, cnt, rec = _select(layer, search, bucket_records=True)
    args = (G["Q"], G["K"], G["V"], G["q_pos"], lr, cnt, layer["cache"], cfg.k, cfg.n_sinks, cfg.window)
    a = lsa.sparse_attend_bucket_major(*args)
    b = lsa.sparse_attend_bucket_major(*args, bucket_records=rec)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_records_that_do_not_match_their_row_use_the_row(layer):
    cfg, G = layer["cfg"], layer["G"]
    lr, cnt, (recs, rcnt) = _select(layer, "flat", bucket_records=True)
    args = (G["Q"], G["K"], G["V"], G["q_pos"], lr, cnt, layer["cache"], cfg.k, cfg.n_sinks, cfg.window)
    ref = lsa.sparse_attend_bucket_major(*args)
    rc = rcnt[0].cpu().numpy()
    rows = np.argwhere(rc > 2)
    rng = np.random.default_rng(9)
    pick = rows[rng.choice(len(rows), size=60, replace=False)]
    bad = recs.clone()
    for x, (i, g) in enumerate(pick):
        if x % 3 == 0:
            bad[0, i, g, 1, 1] ^= 1 << 30                                      # a key more or less
        elif x % 3 == 1:
            bad[0, i, g, 0, 0] = 0x3FFFFFFF                                    # a bucket beyond every block
        else:
            bad[0, i, g, 2, 1] = 0                                             # an empty mask
            bad[0, i, g, 2, 2] = 0
    out = lsa.sparse_attend_bucket_major(*args, bucket_records=(bad, rcnt))
    torch.cuda.synchronize()
    touched = torch.zeros(cfg.T, dtype=torch.bool)
    touched[torch.from_numpy(pick[:, 0])] = True
    d = (out.float() - ref.float()).abs()[0]                                   # [n_q, H_q, d]
    assert torch.equal(out[0][~touched.to(DEV)], ref[0][~touched.to(DEV)])
    print(f"[rec] rows sent to the list path: max diff {float(d.max()):.3e}", flush=True)
    assert float(d.max()) <= tol_for("bf16")


@pytest.mark.parametrize("search", ["flat", "tree"])
def test_skipped_lists_leave_recorded_rows_unwritten_and_the_attention_unchanged(layer, search):
    cfg, G = layer["cfg"], layer["G"]
    lr, cnt, rec = _select(layer, search, bucket_records=True)
    B, n_q, H_kv, k = lr.shape
    lr_s = torch.full_like(lr, -7)
    cnt_s = torch.empty_like(cnt)
    recs_s, rcnt_s = torch.empty_like(rec[0]), torch.empty_like(rec[1])
    _select(layer, search, bucket_records=True, skip_recorded_lists=True, out=(lr_s, cnt_s, recs_s, rcnt_s))
    torch.cuda.synchronize()
    assert torch.equal(cnt_s, cnt) and torch.equal(rcnt_s, rec[1])
    has = rec[1] >= 0
    assert bool((lr_s[has] == -7).all())                     # recorded rows: no list written
    assert torch.equal(lr_s[~has], lr[~has])                # the other rows: their lists
    args = (G["Q"], G["K"], G["V"], G["q_pos"])
    tail = (layer["cache"], cfg.k, cfg.n_sinks, cfg.window)
    a = lsa.sparse_attend_bucket_major(*args, lr, cnt, *tail)
    b = lsa.sparse_attend_bucket_major(*args, lr_s, cnt_s, *tail, bucket_records=(recs_s, rcnt_s))
    torch.cuda.synchronize()
    assert torch.equal(a, b)
