"""Hand the generated tensors to the oracle as numpy arrays (bf16 as raw bits)."""
import numpy as np
import torch


def _np(x):
    if x is None:
        return None
    x = x.detach().cpu()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16)
    return x.numpy()


def arrays_of(inp, use_fp32_originals=False):
    wl = inp.wl
    a = dict(q8=_np(inp.q8), q_scale=_np(inp.q_scale), w=_np(inp.w), k8=_np(inp.k8),
             k_scale=_np(inp.k_scale), q=_np(inp.q), kv=_np(inp.kv), v=_np(inp.v),
             seq_lens=list(inp.seq_lens_host), q_start=inp.q_start_host,
             block_table=_np(inp.block_table), block_size=wl.block_size if inp.paged else 0,
             k=wl.k, scale=wl.scale, D_v=wl.D_v)
    if use_fp32_originals:
        a.update(q_f=_np(inp.q_f32), kv_f=_np(inp.kv_f32), v_f=_np(inp.v_f32))
    return a
