"""The allocation-free indexer entry point (dsa_index_topk_noalloc) against dsa_index_topk with a
workspace, through the C ABI: bit-identical indices on two calls in a row, the second with a smaller
input (fewer tokens, two documents, another k), so that it runs on the scratch the first call left."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import dsa_indexer_top_index_amd as dsa
import testgen as tg
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _both(cfg, q_begin=0, q_end=0):
    print(f"[gpu] noalloc vs workspace indexer: {cfg.name} T={cfg.T} docs={cfg.n_docs} k={cfg.topk} "
          f"rows [{q_begin}, {q_end or cfg.T})", flush=True)
    sys.stdout.flush()
    inp = tg.make_inputs(cfg)
    dev = gu.to_device(inp)
    shape = gu.shape_of(cfg, dev.get("cu_seqlens"), q_begin, q_end)
    rows = (q_end or cfg.T) - q_begin
    sl = slice(q_begin, q_begin + rows)
    q_I, w = dev["q_I"][sl].contiguous(), dev["w"][sl].contiguous()
    ws = dsa.alloc_workspace(shape)
    ref = torch.empty((rows, cfg.topk), dtype=torch.int32, device="cuda")
    got = torch.full((rows, cfg.topk), -7, dtype=torch.int32, device="cuda")
    dsa.dsa_index_topk(shape, q_I, dev["k_I"], w, ref, ws)
    dsa.dsa_index_topk_noalloc(shape, q_I, dev["k_I"], w, got)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


def test_noalloc_matches_workspace_entry_point_two_calls():
    first = tg.get_config("t8192")
    second = tg.Config("noalloc-small", 51, [1300, 903], topk=512, H=96, H_I=64, d_I=128, w_scale=1 / 8,
                       q_std=1 / 24, W_UV_std=0.02)
    for cfg in (first, second):
        ref, got = _both(cfg)
        assert np.array_equal(ref, got), f"{cfg.name}: {np.sum(ref != got)} entries differ"
    # a row range of the second input, and the 16-head, 4x64 indexer shape
    ref, got = _both(second, q_begin=700, q_end=2000)
    assert np.array_equal(ref, got)
    tiny = tg.get_config("tiny")
    ref, got = _both(tiny)
    assert np.array_equal(ref, got)

