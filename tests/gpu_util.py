"""Moves a workloads.Problem to the GPU as torch tensors for the binding (test helper)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import workloads as W


def dev(prob: W.Problem, device="cuda"):
    """Returns dict(q, k, w, q_pos, k_len, k_scale, q_scale, wk) of device tensors holding the
    same bytes."""
    if prob.q_dtype == W.BF16:
        q = torch.from_numpy(prob.q.view(np.int16)).view(torch.bfloat16)
    elif prob.q_dtype == W.FP8_E4M3:
        q = torch.from_numpy(prob.q).view(torch.float8_e4m3fn)
    else:
        q = torch.from_numpy(prob.q)
    if prob.k_dtype == W.BF16:
        k = torch.from_numpy(prob.k.view(np.int16)).view(torch.bfloat16)
    elif prob.k_dtype == W.FP8_E4M3:
        k = torch.from_numpy(prob.k).view(torch.float8_e4m3fn)
    else:
        k = torch.from_numpy(prob.k)
    out = dict(q=q.to(device), k=k.to(device), w=torch.from_numpy(prob.w).to(device),
               q_pos=torch.from_numpy(prob.q_pos).to(device),
               k_len=torch.from_numpy(prob.k_len).to(device), k_scale=None)
    if prob.k_scale is not None:
        out["k_scale"] = torch.from_numpy(prob.k_scale).to(device)
    out["q_scale"] = None
    if getattr(prob, "q_scale", None) is not None:
        out["q_scale"] = torch.from_numpy(prob.q_scale).to(device)
    out["wk"] = None
    if getattr(prob, "wk", None) is not None:
        out["wk"] = torch.from_numpy(prob.wk.view(np.int16)).view(torch.bfloat16).to(device)
    return out


def say(*a):
    """Print and flush (names the case before a GPU step)."""
    print(*a, flush=True)
    sys.stdout.flush()
