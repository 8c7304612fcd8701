"""Move a host workload to GPU tensors and back (torch plumbing only)."""
from __future__ import annotations

import dataclasses

import numpy as np


def np_to_torch(a: np.ndarray, kv_dtype: str, device):
    """Host storage array -> device tensor of the KV dtype (bits preserved)."""
    import torch
    if kv_dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def torch_to_np(t, kv_dtype: str) -> np.ndarray:
    """Device tensor -> host storage array (raw uint16 for bf16, float32 otherwise)."""
    import torch
    if kv_dtype == "bf16":
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


@dataclasses.dataclass
class DeviceWorkload:
    k_cache: object
    v_cache: object
    q: object
    k_new: object
    v_new: object
    slot_mapping: object
    block_tables: object
    context_lens: object
    out: object


def upload(w, device="cuda:0") -> DeviceWorkload:
    import torch
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
    return DeviceWorkload(
        k_cache=np_to_torch(w.k_cache, w.kv_dtype, device),
        v_cache=np_to_torch(w.v_cache, w.kv_dtype, device),
        q=np_to_torch(w.q, w.kv_dtype, device),
        k_new=np_to_torch(w.k_new, w.kv_dtype, device),
        v_new=np_to_torch(w.v_new, w.kv_dtype, device),
        slot_mapping=i32(w.slot_mapping),
        block_tables=i32(w.block_tables),
        context_lens=i32(w.context_lens),
        out=torch.full((w.num_seqs, w.num_heads, w.head_dim), float("nan"), dtype=torch.float32,
                       device=device),
    )
