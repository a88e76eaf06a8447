"""The allocation-free attention entry point (lsa_sparse_attend_noalloc) against lsa_sparse_attend with a
caller workspace: the same kernels on the same inputs, so the outputs must be identical bit for bit; two
calls in a row (the second smaller) share the library's scratch array; a call whose split-key partials
would not fit is refused before anything is queued."""

import ctypes
import math

import numpy as np
import pytest
import torch

import sparse_attention_indexing_latent_amd as lsa
from sparse_attention_indexing_latent_amd import _lib
from synth import get_config, layer_inputs, random_lr_lists

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _decode_case(B, H_kv, H_q, T, seed):
    """B sequences, one query each at position T (K/V rows 0..T), with synthetic long-range lists."""
    cfg = get_config(2, T=T, B=B, H_kv=H_kv, H_q=H_q, n_topics=32, k=512, window=256)
    qp = torch.full((B, 1), T, dtype=torch.int64)
    inp = layer_inputs(cfg, seed=seed, T_cap=T + 1, q_positions=qp)
    idx, cnt = random_lr_lists(cfg, qp, seed=seed)
    G = {k: inp[k].to(DEV).contiguous() for k in ("K", "V", "Q", "q_pos")}
    return cfg, G, idx.to(DEV), cnt.to(DEV)


def _noalloc_ctypes(cfg, G, idx, cnt, O):
    """The C entry point called directly through ctypes."""
    B, n_q, H_q, d = G["Q"].shape
    _, H_kv, t_cap, _ = G["K"].shape
    layout = lsa.make_layout(d, H_kv, H_q, G["Q"].dtype)
    scfg = lsa.select_cfg(cfg.k, cfg.n_sinks, cfg.window)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = _lib.lib().lsa_sparse_attend_noalloc(ctypes.byref(layout), ctypes.byref(scfg), p(G["Q"]), p(G["K"]),
                                             p(G["V"]), t_cap, cfg.T, p(G["q_pos"]), B, n_q, p(idx), p(cnt),
                                             ctypes.c_float(1 / math.sqrt(d)), p(O),
                                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def test_noalloc_equals_workspace_call_twice():
    big = _decode_case(B=12, H_kv=4, H_q=20, T=16384, seed=3)      # 48 units: split over their key lists
    small = _decode_case(B=3, H_kv=2, H_q=10, T=10240, seed=4)     # 6 units: more splits each, a smaller input
    for cfg, G, idx, cnt in (big, small):
        assert lsa.attend_workspace_bytes(G["Q"], G["K"].shape[1], cfg.k, cfg.window) > 0
        ref = lsa.sparse_attend(G["Q"], G["K"], G["V"], G["q_pos"], idx, cnt, cfg.T, cfg.k, cfg.n_sinks, cfg.window)
        O = torch.full_like(G["Q"], float("nan"))
        assert _noalloc_ctypes(cfg, G, idx, cnt, O) == 0, _lib.lib().lsa_last_error()
        torch.cuda.synchronize()
        print(f"[noalloc] B={G['Q'].shape[0]} H_q={G['Q'].shape[2]}: bit-identical "
              f"{bool(torch.equal(O, ref))}", flush=True)
        assert torch.equal(O, ref)
    # and once more on the first input, after the smaller call left its contents in the array
    cfg, G, idx, cnt = big
    ref = lsa.sparse_attend(G["Q"], G["K"], G["V"], G["q_pos"], idx, cnt, cfg.T, cfg.k, cfg.n_sinks, cfg.window)
    O = lsa.sparse_attend_noalloc(G["Q"], G["K"], G["V"], G["q_pos"], idx, cnt, cfg.T, cfg.k, cfg.n_sinks, cfg.window)
    torch.cuda.synchronize()
    assert torch.equal(O, ref)


def test_noalloc_refuses_more_than_its_scratch():
    # G = 8, d = 128, 128 units split 8 ways: 4.26 MB of partials > 4 MiB
    layout = lsa.make_layout(128, 1, 8, torch.bfloat16)
    scfg = lsa.select_cfg(2048, 4, 1024)
    fake = ctypes.c_void_p(0x1000)
    st = _lib.lib().lsa_sparse_attend_noalloc(ctypes.byref(layout), ctypes.byref(scfg), fake, fake, fake, 8192, 8192,
                                             fake, 128, 1, fake, fake, ctypes.c_float(0.1), fake, None)
    assert st == 5, st
    assert b"4194304" in _lib.lib().lsa_last_error()
