"""Checkpoint and resume of the compressed optimizer state.

The state of the compressed phase lives in caller-owned device buffers: the
worker and server error states with their chunk scales, the packed global
momentum, the parameters, the frozen and fresh variances, the previous global
momentum and the per-layer tables. A checkpoint writes each buffer as a raw
little-endian dump next to a JSON manifest (name, dtype, shape, byte count)
and a free-form ``meta`` record (step counter, seeds, hyper-parameters).
Loading reads the dumps with numpy, so nothing in the files is executed, and
checks every size against the manifest.

    save(path, {"ef": t, ...}, meta={"t": 17})
    tensors, meta = load(path, device)
"""

from __future__ import annotations

import json
import os
from typing import Dict, Mapping, Optional, Tuple

import numpy as np
import torch

MANIFEST = "manifest.json"
FORMAT = 1

_DTYPES = {
    torch.float32: "<f4",
    torch.float64: "<f8",
    torch.int32: "<i4",
    torch.int64: "<i8",
    torch.int8: "|i1",
    torch.uint8: "|u1",
}
_TORCH = {v: k for k, v in _DTYPES.items()}


def save(path: str, tensors: Mapping[str, Optional[torch.Tensor]],
         meta: Optional[dict] = None) -> None:
    """Write every non-None tensor of ``tensors`` under ``path`` (a directory,
    created if needed). The copies to the host are synchronous, so the
    files hold the values the stream had reached when ``save`` was called."""
    os.makedirs(path, exist_ok=True)
    entries = {}
    for name, t in tensors.items():
        if t is None:
            continue
        if t.dtype not in _DTYPES:
            raise TypeError(f"{name}: dtype {t.dtype} has no checkpoint encoding")
        a = t.detach().contiguous().cpu().numpy()
        dt = np.dtype(_DTYPES[t.dtype])
        fname = f"{name}.bin"
        a.astype(dt, copy=False).tofile(os.path.join(path, fname))
        entries[name] = {"file": fname, "dtype": _DTYPES[t.dtype], "shape": list(a.shape),
                         "bytes": int(a.size) * dt.itemsize}
    record = {"format": FORMAT, "tensors": entries, "meta": dict(meta or {})}
    tmp = os.path.join(path, MANIFEST + ".tmp")
    with open(tmp, "w") as f:
        json.dump(record, f, indent=1, sort_keys=True)
    os.replace(tmp, os.path.join(path, MANIFEST))


def load(path: str, device) -> Tuple[Dict[str, torch.Tensor], dict]:
    """Read a checkpoint written by ``save``; tensors are placed on ``device``."""
    with open(os.path.join(path, MANIFEST)) as f:
        record = json.load(f)
    if record.get("format") != FORMAT:
        raise ValueError(f"unknown checkpoint format {record.get('format')!r}")
    out = {}
    for name, e in record["tensors"].items():
        if e["dtype"] not in _TORCH:
            raise ValueError(f"{name}: unknown dtype {e['dtype']!r}")
        fname = os.path.join(path, e["file"])
        if os.path.basename(e["file"]) != e["file"]:
            raise ValueError(f"{name}: file name {e['file']!r} leaves the checkpoint")
        dt = np.dtype(e["dtype"])
        count = int(np.prod(e["shape"], dtype=np.int64))
        if os.path.getsize(fname) != e["bytes"] or e["bytes"] != count * dt.itemsize:
            raise ValueError(f"{name}: {fname} does not hold {e['shape']} x {e['dtype']}")
        a = np.fromfile(fname, dtype=dt, count=count).reshape(e["shape"])
        out[name] = torch.from_numpy(a.astype(dt.newbyteorder("="), copy=False)).to(device)
    return out, record["meta"]
