"""Device-side helpers for the GPU tests, the smoke check and the benchmark (no method arithmetic)."""
from __future__ import annotations

import numpy as np
import torch

import dsa_indexer_top_index_amd as dsa


def bf16_np_to_tensor(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def bf16_tensor_to_f32(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def to_device(inp: dict, device="cuda") -> dict:
    d = {}
    for k, v in inp.items():
        if k == "cu_seqlens":
            d[k] = torch.from_numpy(np.ascontiguousarray(v, dtype=np.int32)).to(device)
        else:
            d[k] = bf16_np_to_tensor(v, device)
    return d


def shape_of(cfg, cu_dev=None, q_begin=0, q_end=0, topk=None):
    multi = cfg.n_docs > 1
    return dsa.make_shape(cfg.T, topk or cfg.topk, cfg.H_I, cfg.d_I, cfg.H,
                          cu_seqlens=[int(x) for x in cfg.cu_seqlens] if multi else None,
                          cu_seqlens_dev=cu_dev if multi else None, q_begin=q_begin, q_end=q_end,
                          ln_eps=cfg.ln_eps, softmax_scale=cfg.softmax_scale)


def run_fused(cfg, dev, q_begin=0, q_end=0, with_lse=False, ws=None):
    shape = shape_of(cfg, dev.get("cu_seqlens"), q_begin, q_end)
    rows = (q_end or cfg.T) - q_begin
    ws = dsa.alloc_workspace(shape) if ws is None else ws
    sl = slice(q_begin, q_begin + rows)
    topk_idx = torch.empty((rows, cfg.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((rows, cfg.H, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((rows, cfg.H), dtype=torch.float32, device="cuda") if with_lse else None
    dsa.dsa_fused_fwd(shape, dev["q_I"][sl].contiguous(), dev["k_I"], dev["w"][sl].contiguous(),
                      dev["q"][sl].contiguous(), dev["kv"], dev["W_UV"], dev["gate"][sl].contiguous(),
                      topk_idx, out, ws, lse=lse)
    return {"topk_idx": topk_idx, "out": out, "lse": lse, "ws": ws, "shape": shape}


def device_inputs(cfg, chunk_rows: int = 4096):
    """Key-side tensors on host (for the oracle) and every tensor on the device. Query-side tensors
    are drawn in row chunks straight into device memory, so host memory stays bounded at T=131072."""
    import testgen as tg

    keys = tg.key_side(cfg)
    dev = {k: bf16_np_to_tensor(v) for k, v in keys.items()}
    T = cfg.T
    specs = [("q_I", tg.TAG_QI, cfg.H_I * cfg.d_I, cfg.q_I_std, tg.normal_bf16, (cfg.H_I, cfg.d_I)),
             ("w", tg.TAG_W, cfg.H_I, cfg.w_scale, tg.uniform_bf16, (cfg.H_I,)),
             ("q", tg.TAG_Q, cfg.H * tg.D_L, cfg.q_std, tg.normal_bf16, (cfg.H, tg.D_L)),
             ("gate", tg.TAG_GATE, cfg.H, cfg.gate_std, tg.normal_bf16, (cfg.H,))]
    for name, tag, per_row, scale, fn, tail in specs:
        t = torch.empty((T, per_row), dtype=torch.bfloat16, device="cuda")
        for r0 in range(0, T, chunk_rows):
            n = min(chunk_rows, T - r0)
            arr = fn(cfg.seed, tag, r0 * per_row, n * per_row, scale).reshape(n, per_row)
            t[r0:r0 + n] = bf16_np_to_tensor(arr)
        dev[name] = t.view(T, *tail)
    dev["cu_seqlens"] = torch.from_numpy(cfg.cu_seqlens).to("cuda")
    return keys, dev
