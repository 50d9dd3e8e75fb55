"""Upload a synthetic workload to the GPU and allocate the step's outputs."""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

from . import workloads as W


@dataclasses.dataclass
class DeviceStep:
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    kv_start: torch.Tensor
    kv_len: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    k_prefix: Optional[torch.Tensor]
    v_prefix: Optional[torch.Tensor]
    out: torch.Tensor
    target_logits: torch.Tensor
    draft_logits: torch.Tensor
    draft_tokens: torch.Tensor
    u_accept: torch.Tensor
    u_sample: torch.Tensor
    n_accepted: torch.Tensor
    out_tokens: torch.Tensor
    tokens_packed: torch.Tensor
    cu_tokens: torch.Tensor
    status: torch.Tensor


def kv_tensor(a: np.ndarray, device) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> torch.bfloat16; float32 stays float32."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_device(w: W.Workload, device, logits_dtype=torch.float32) -> DeviceStep:
    c = w.cfg
    B, K = c.B, c.K
    q = kv_tensor(w.q, device)
    kp = kv_tensor(w.k_prefix, device) if w.k_prefix is not None else None
    vp = kv_tensor(w.v_prefix, device) if w.v_prefix is not None else None
    return DeviceStep(
        q=q,
        k_cache=kv_tensor(w.k_cache, device),
        v_cache=kv_tensor(w.v_cache, device),
        kv_start=torch.from_numpy(w.kv_start).to(device),
        kv_len=torch.from_numpy(w.kv_len).to(device),
        k_new=kv_tensor(w.k_new, device),
        v_new=kv_tensor(w.v_new, device),
        k_prefix=kp,
        v_prefix=vp,
        out=torch.empty_like(q),
        target_logits=torch.from_numpy(w.target_logits).to(device).to(logits_dtype),
        draft_logits=torch.from_numpy(w.draft_logits).to(device).to(logits_dtype),
        draft_tokens=torch.from_numpy(w.draft_tokens).to(device),
        u_accept=torch.from_numpy(w.u_accept).to(device),
        u_sample=torch.from_numpy(w.u_sample).to(device),
        n_accepted=torch.full((B,), -7, dtype=torch.int32, device=device),
        out_tokens=torch.full((B, K + 1), -7, dtype=torch.int32, device=device),
        tokens_packed=torch.full((B * (K + 1),), -1, dtype=torch.int32, device=device),
        cu_tokens=torch.zeros(B + 1, dtype=torch.int32, device=device),
        status=torch.zeros(1, dtype=torch.int32, device=device),
    )


@dataclasses.dataclass
class RaggedDeviceStep(DeviceStep):
    cu_q: Optional[torch.Tensor] = None
    cu_q_host: Optional[list] = None


def ragged_to_device(rw: W.RaggedWorkload, device, logits_dtype=torch.float32) -> RaggedDeviceStep:
    """Device tensors of a ragged-draft-length workload (rows packed by cu_q)."""
    w = rw.base
    B = w.cfg.B
    NT = int(rw.cu_q[-1])
    q = kv_tensor(rw.q, device)
    kp = kv_tensor(w.k_prefix, device) if w.k_prefix is not None else None
    vp = kv_tensor(w.v_prefix, device) if w.v_prefix is not None else None
    return RaggedDeviceStep(
        q=q,
        k_cache=kv_tensor(w.k_cache, device),
        v_cache=kv_tensor(w.v_cache, device),
        kv_start=torch.from_numpy(w.kv_start).to(device),
        kv_len=torch.from_numpy(w.kv_len).to(device),
        k_new=kv_tensor(rw.k_new, device),
        v_new=kv_tensor(rw.v_new, device),
        k_prefix=kp,
        v_prefix=vp,
        out=torch.empty_like(q),
        target_logits=torch.from_numpy(rw.target_logits).to(device).to(logits_dtype),
        draft_logits=torch.from_numpy(rw.draft_logits).to(device).to(logits_dtype),
        draft_tokens=torch.from_numpy(rw.draft_tokens).to(device),
        u_accept=torch.from_numpy(rw.u_accept).to(device),
        u_sample=torch.from_numpy(w.u_sample).to(device),
        n_accepted=torch.full((B,), -7, dtype=torch.int32, device=device),
        out_tokens=torch.full((NT,), -7, dtype=torch.int32, device=device),
        tokens_packed=torch.full((NT,), -1, dtype=torch.int32, device=device),
        cu_tokens=torch.zeros(B + 1, dtype=torch.int32, device=device),
        status=torch.zeros(1, dtype=torch.int32, device=device),
        cu_q=torch.from_numpy(rw.cu_q).to(device),
        cu_q_host=[int(x) for x in rw.cu_q],
    )
