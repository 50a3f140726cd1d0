"""Checkpoint files on the host: round trip of every supported dtype, the
manifest, and refusal of damaged or escaping entries; the group and LAMB
state round trip through ``from_state`` (host tensors, no kernel runs)."""

import json

import numpy as np
import pytest
import torch

from momentum_compression_amd import checkpoint as ck
from momentum_compression_amd.state import AdamWarmup, LambState, LambWarmup, OneBitGroup


def _tensors():
    g = torch.Generator().manual_seed(3)
    return {
        "f32": torch.randn(7, 33, generator=g),
        "f64": torch.randn(5, generator=g, dtype=torch.float64),
        "i32": torch.randint(-2**31, 2**31 - 1, (64,), generator=g, dtype=torch.int32),
        "i64": torch.tensor([0, -1, 2**62, -2**62], dtype=torch.int64),
        "u8": torch.randint(0, 256, (3, 4), generator=g, dtype=torch.uint8),
        "i8": torch.randint(-128, 128, (9,), generator=g, dtype=torch.int8),
        "scalar": torch.tensor(1.5),
        "empty": torch.zeros(0, 4),
    }


def test_round_trip_every_dtype(tmp_path):
    t = _tensors()
    ck.save(str(tmp_path), {**t, "absent": None}, meta={"t": 17, "seed": 2**40 + 3})
    back, meta = ck.load(str(tmp_path), "cpu")
    assert meta == {"t": 17, "seed": 2**40 + 3}
    assert set(back) == set(t)
    for k, v in t.items():
        assert back[k].dtype == v.dtype and back[k].shape == v.shape
        assert torch.equal(back[k], v), k
    man = json.load(open(tmp_path / ck.MANIFEST))
    assert man["format"] == ck.FORMAT
    assert man["tensors"]["f32"] == {"file": "f32.bin", "dtype": "<f4", "shape": [7, 33],
                                     "bytes": 7 * 33 * 4}
    # raw little-endian: the file is the array's bytes in that order
    raw = np.fromfile(tmp_path / "i64.bin", dtype="<i8")
    assert list(raw) == [0, -1, 2**62, -2**62]


def test_damaged_files_are_refused(tmp_path):
    ck.save(str(tmp_path), {"a": torch.arange(10, dtype=torch.float32)})
    with open(tmp_path / "a.bin", "r+b") as f:
        f.truncate(36)
    with pytest.raises(ValueError):
        ck.load(str(tmp_path), "cpu")
    ck.save(str(tmp_path), {"a": torch.arange(10, dtype=torch.float32)})
    man = json.load(open(tmp_path / ck.MANIFEST))
    man["tensors"]["a"]["file"] = "../a.bin"
    json.dump(man, open(tmp_path / ck.MANIFEST, "w"))
    with pytest.raises(ValueError):
        ck.load(str(tmp_path), "cpu")
    man["tensors"]["a"]["file"] = "a.bin"
    man["format"] = 99
    json.dump(man, open(tmp_path / ck.MANIFEST, "w"))
    with pytest.raises(ValueError):
        ck.load(str(tmp_path), "cpu")


@pytest.mark.parametrize("keep_prev", [False, True])
def test_group_and_lamb_state_round_trip(tmp_path, keep_prev):
    N, n = 4096, 4
    off = torch.tensor([0, 100, 100, 3000, N], dtype=torch.int64)
    k = torch.tensor([1.0, 2.0, 0.5, 4.0])
    grp = OneBitGroup(N, n, torch.device("cpu"), clip=2.0, reset_interval=2000, seg_off=off,
                      seg_k=k, keep_prev=keep_prev)
    assert ("sv_bits_prev" in grp.state_dict()) == keep_prev
    g = torch.Generator().manual_seed(5)
    for name in grp._state_names():
        buf = getattr(grp, name)
        if buf.dtype == torch.float32:
            buf.copy_(torch.randn(buf.shape, generator=g))
        else:
            buf.copy_(torch.randint(-2**31, 2**31 - 1, buf.shape, generator=g, dtype=buf.dtype))
    S = off.numel() - 1
    st = LambState.create(torch.randn(N, generator=g), torch.rand(N, generator=g),
                          torch.randn(N, generator=g), off, torch.rand(S, generator=g))
    st.v_fresh.copy_(torch.rand(N, generator=g))
    st.r.copy_(torch.rand(S, generator=g))
    st.c.copy_(torch.rand(S, generator=g))
    ck.save(str(tmp_path / "g"), grp.state_dict(), meta={"t": 5, "group": grp.config()})
    ck.save(str(tmp_path / "l"), st.state_dict())
    tg, meta = ck.load(str(tmp_path / "g"), "cpu")
    grp2 = OneBitGroup.from_state(tg, meta["group"], torch.device("cpu"))
    assert grp2.config() == grp.config() and meta["t"] == 5
    for name, v in grp.state_dict().items():
        w = grp2.state_dict()[name]
        assert (v is None and w is None) or torch.equal(v, w), name
    tl, _ = ck.load(str(tmp_path / "l"), "cpu")
    st2 = LambState.from_state(tl)
    for name, v in st.state_dict().items():
        assert torch.equal(v, getattr(st2, name)), name
    bad = dict(tg)
    bad["ef"] = bad["ef"][:, :64]
    with pytest.raises(ValueError):
        OneBitGroup.from_state(bad, meta["group"], torch.device("cpu"))


def test_warmup_state_round_trip(tmp_path):
    g = torch.Generator().manual_seed(9)
    N = 1000
    off = torch.tensor([0, 10, 10, 600, N], dtype=torch.int64)
    aw = AdamWarmup.create(torch.randn(N, generator=g))
    aw.m.copy_(torch.randn(N, generator=g))
    aw.v.copy_(torch.rand(N, generator=g))
    lw = LambWarmup.create(torch.randn(N, generator=g), off)
    lw.m.copy_(torch.randn(N, generator=g))
    lw.v.copy_(torch.rand(N, generator=g))
    lw.c.copy_(torch.rand(4, generator=g))
    lw.c_avg.copy_(torch.rand(4, generator=g))
    lw.steps = 7
    ck.save(str(tmp_path / "a"), aw.state_dict())
    ck.save(str(tmp_path / "l"), lw.state_dict(), meta={"steps": lw.steps})
    ta, _ = ck.load(str(tmp_path / "a"), "cpu")
    aw2 = AdamWarmup.from_state(ta)
    for k, v in aw.state_dict().items():
        assert torch.equal(v, aw2.state_dict()[k]), k
    tl, meta = ck.load(str(tmp_path / "l"), "cpu")
    lw2 = LambWarmup.from_state(tl, meta["steps"])
    assert lw2.steps == 7
    for k, v in lw.state_dict().items():
        assert torch.equal(v, lw2.state_dict()[k]), k


def test_keep_prev_group_layout_and_capture_refused():
    """A keep_prev group holds its scales as the two halves of one buffer of
    2n (this step's, then the previous step's), which the server's
    ONEBIT_KEEP_PREV call takes whole, and refuses graph capture (its word
    buffers alternate, a graph would replay fixed pointers)."""
    N, n = 4096, 4
    grp = OneBitGroup(N, n, torch.device("cpu"), keep_prev=True)
    assert grp._sv_scales2.numel() == 2 * n
    assert grp.sv_scales.data_ptr() == grp._sv_scales2.data_ptr()
    assert grp.sv_scales_prev.data_ptr() == grp._sv_scales2.data_ptr() + 4 * n
    assert grp.sv_bits_prev.shape == grp.sv_bits.shape
    assert grp.config()["keep_prev"] is True
    with pytest.raises(ValueError):
        grp.capture_step(None, None, None, 1e-3, 1e-6)
    plain = OneBitGroup(N, n, torch.device("cpu"))
    assert not hasattr(plain, "sv_bits_prev") and plain.config()["keep_prev"] is False
