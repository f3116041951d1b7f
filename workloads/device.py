"""Device-side staging of the generated inputs (torch): page pools holding the
KV that exists before a workload's first call, and the row tensors a call
compacts.  Input construction only; nothing here computes the method."""
from __future__ import annotations

import numpy as np
import torch

from . import PAGE_SIZE, paged_given_cache


def torch_dtype(wl):
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def stored_to_tensor(x: np.ndarray, device="cuda") -> torch.Tensor:
    """Storage form (uint16 bf16 bits or float32) to a device tensor."""
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def make_caches(wl, device="cuda"):
    """Page pools [num_pages, Hkv, 16, D]: zero, plus the KV that exists before
    the first call - drawn on the device by torch's seeded generator when the
    workload asks for it (too large to draw on the host), else the workload's
    given cache."""
    shape = (wl.num_pages, wl.Hkv, PAGE_SIZE, wl.D)
    if wl.device_cache_seed is not None:
        kc = torch.zeros(shape, dtype=torch_dtype(wl), device=device)
        vc = torch.zeros_like(kc)
        gen = torch.Generator(device=device)
        gen.manual_seed(int(wl.device_cache_seed))
        for pid in sorted(wl.device_cache_ctx):
            c = wl.device_cache_ctx[pid]
            pg = torch.from_numpy(wl.prompt_pages[pid].astype(np.int64)).to(device)
            lp = torch.arange(c, device=device)
            page, off = pg[lp // PAGE_SIZE], lp % PAGE_SIZE
            K = torch.randn((c, wl.Hkv, wl.D), generator=gen, device=device).to(kc.dtype)
            V = torch.randn((c, wl.Hkv, wl.D), generator=gen, device=device).to(kc.dtype)
            kc[page, :, off, :] = K
            vc[page, :, off, :] = V
        return kc, vc
    kh, vh = paged_given_cache(wl)
    return stored_to_tensor(kh, device), stored_to_tensor(vh, device)


def row_sources(call, device="cuda"):
    """(name, tensor) of every row tensor a call compacts."""
    rows = [("hidden", stored_to_tensor(call.hidden, device)),
            ("positions", torch.from_numpy(call.positions.astype(np.int32)).to(device)),
            ("slot_mapping", torch.from_numpy(call.slot_mapping.astype(np.int32)).to(device))]
    for name in sorted(call.extra):
        rows.append((name, stored_to_tensor(call.extra[name], device)))
    return rows
