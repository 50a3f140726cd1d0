"""Write tests/golden/oracle_regression.json: SHA-256 digests (and the first
values) of the oracle's outputs on small seeded inputs.

These are regression values of the oracle itself, not pins to the pages:
any change to the oracle's arithmetic changes a digest, so it cannot pass
unnoticed.  The script calls only oracle/ (and numpy's seeded generator for
the inputs).

    python tests/golden/make_golden.py
"""

from __future__ import annotations

import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import int8 as I  # noqa: E402
from oracle import onebit as O  # noqa: E402
from oracle import optim as P  # noqa: E402
from oracle import philox as PH  # noqa: E402
from oracle import warmup as W  # noqa: E402

F32 = np.float32
OUT = os.path.join(HERE, "oracle_regression.json")


def _normal(seed, shape, scale):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(F32)


def _digest(a) -> dict:
    a = np.ascontiguousarray(np.asarray(a))
    le = a.astype(a.dtype.newbyteorder("<"), copy=False)
    head = [float(v) if a.dtype.kind == "f" else int(v) for v in a.ravel()[:4]]
    return {"dtype": str(a.dtype), "shape": list(a.shape),
            "sha256": hashlib.sha256(le.tobytes()).hexdigest(), "head": head}


def cases() -> dict:
    out = {}
    n, N = 4, 1024
    off = np.array([0, 100, 612, 612, N], dtype=np.int64)
    k = np.array([0.5, 2.0, 3.0, 4.0], dtype=F32)
    k_el = O.per_element_k(off, k)
    m = _normal(1, (n, N), 1e-3)
    e = _normal(2, (n, N), 1e-4)
    w = O.worker_compress(m, e, clip=2.5e-3, k=k_el)
    out["worker_compress"] = {key: _digest(w[key]) for key in ("gc", "bits", "s", "e")}
    E = _normal(3, N, 1e-4)
    sv = O.server_reduce(w["bits"], w["s"], E)
    out["server_reduce"] = {key: _digest(sv[key]) for key in ("avg", "g2", "bits", "S", "E")}
    rho = O.per_element_k(off, np.array([0.5, 1.0, 2.0, 1.5], dtype=F32))
    sv2 = O.server_reduce(w["bits"], w["s"], E, err_ratio=rho)
    out["server_reduce_step_ratio"] = {key: _digest(sv2[key]) for key in ("g2", "S", "E")}
    mbar = O.decompress(sv["bits"], sv["S"], k=k_el)
    out["decompress"] = {"m": _digest(mbar)}
    out["local_momentum"] = {"m": _digest(O.local_momentum(_normal(4, (n, N), 1e-3), mbar, 0.9))}
    x = _normal(5, N, 0.02)
    v = np.abs(_normal(6, N, 1e-6)) + F32(1e-8)
    out["adam_frozen_step"] = {"x": _digest(P.adam_frozen_step(x, mbar, v, 6e-5, 1e-6))}
    S = len(off) - 1
    c_avg = np.array([1.0, 0.8, 1.2, 0.9], dtype=F32)
    lb = P.lamb_frozen_step(x, mbar, _normal(7, N, 1e-3), v.copy(), v, off, c_avg,
                            np.ones(S, dtype=F32), c_avg.copy(), 1e-3, 1e-6, 0.9, 0.999,
                            0.1, 0.5, 4.0)
    out["lamb_frozen_step"] = {key: _digest(lb[key]) for key in ("x", "v", "R", "r", "c", "err_ratio")}
    g = (np.random.default_rng(8).laplace(0.0, 1e-3, N)).astype(F32)
    ei = _normal(9, N, 1e-5)
    for name, kw in (("int8_sr_block64", dict(block=64)),
                     ("int8_nearest_block256", dict(block=256, rounding="nearest")),
                     ("int8_sr_tensor", dict(block=0))):
        r = I.int8_sr(g, ei, 2**40 + 3, 5, **kw)
        out[name] = {key: _digest(r[key]) for key in ("codes", "scales", "deq", "e")}
    out["philox_uniforms"] = {"u": _digest(PH.uniforms((1 << 32) - 8, 16, 2**40 + 3, 0xFFFFFFF0))}
    gw = _normal(10, N, 1e-3)
    aw = W.adam_warmup_step(x, np.zeros(N, F32), np.zeros(N, F32), gw, 1e-3, 1e-8, 0.9, 0.999)
    out["adam_warmup_step"] = {key: _digest(aw[key]) for key in ("x", "m", "v")}
    lw = W.lamb_warmup_step(x, _normal(11, N, 1e-3), np.abs(_normal(12, N, 1e-6)), gw, off,
                            1e-3, 1e-6, 0.9, 0.999, c_avg=c_avg, beta_c=0.9)
    out["lamb_warmup_step"] = {key: _digest(lw[key]) for key in ("x", "m", "v", "c", "c_avg")}
    out["momentum_scale"] = {"k": _digest(W.momentum_scale(_normal(13, N, 1e-3), off))}
    return out


if __name__ == "__main__":
    with open(OUT, "w") as f:
        json.dump(cases(), f, indent=1, sort_keys=True)
        f.write("\n")
    print(f"wrote {OUT}")
