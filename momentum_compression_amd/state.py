"""Device buffers of one simulated data-parallel group and the calls of one
compressed step, driven through the C ABI.

PyTorch is used only to allocate device memory and to pick the stream; every
element of every step is computed by libonebit's kernels.

Buffers (n workers, N elements per worker row, chunk L = N / n):

    ef        [n, N]    worker error state (last compensated value)
    scales    [n, n]    worker chunk scales s[i][c] (error state, second half)
    bits      [n, N/32] worker sign words
    sv_ef     [N]       server error state
    sv_scales [n]       server chunk scales
    sv_bits   [N/32]    server sign words
    mbar      [N]       decompressed global momentum
    ws        bytes     scratch for the chunk sums and layer maxima
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Mapping, Optional

import torch

from . import onebit as ob


@dataclass
class OneBitGroup:
    N: int
    n: int
    device: torch.device
    clip: float = 0.0
    reset_interval: int = 0
    seg_off: Optional[torch.Tensor] = None  # int64 [S+1] on device
    seg_k: Optional[torch.Tensor] = None    # float32 [S] on device
    unit_scale: bool = False                # unscaled +-1 signs at both levels
    seg_err_ratio: Optional[torch.Tensor] = None  # float32 [S]: step-ratio error factor
    # keep the previous step's server words and scales (sv_bits_prev,
    # sv_scales_prev), so the LAMB step can read m_{t-1} packed: the server
    # writes its words into the older of two buffers (they swap every step;
    # the words are output only), and copies its scales, which are also its
    # error state, to a second half before overwriting them
    keep_prev: bool = False

    def __post_init__(self):
        N, n, dev = self.N, self.n, self.device
        if N % (64 * n):
            raise ValueError("N must be a multiple of 64 * n (pad the buffer)")
        f32 = torch.float32
        self.ef = torch.zeros((n, N), dtype=f32, device=dev)
        self.scales = torch.zeros((n, n), dtype=f32, device=dev)
        self.bits = torch.zeros((n, N // 32), dtype=torch.int32, device=dev)
        self.sv_ef = torch.zeros(N, dtype=f32, device=dev)
        self.sv_scales = torch.zeros(n, dtype=f32, device=dev)
        self.sv_bits = torch.zeros(N // 32, dtype=torch.int32, device=dev)
        self.mbar = torch.zeros(N, dtype=f32, device=dev)
        if self.keep_prev:
            self._sv_scales2 = torch.zeros(2 * n, dtype=f32, device=dev)
            self.sv_scales = self._sv_scales2[:n]
            self.sv_scales_prev = self._sv_scales2[n:]
            self.sv_bits_prev = torch.zeros(N // 32, dtype=torch.int32, device=dev)
        n_seg = self.n_seg
        self.ws = torch.empty(max(256, ob.workspace_bytes(N, n, n_seg)), dtype=torch.uint8, device=dev)

    @property
    def n_seg(self) -> int:
        return 0 if self.seg_off is None else self.seg_off.numel() - 1

    def is_reset(self, t: int) -> bool:
        """Periodic error reset (1-bit Adam article, section 4.1): zero the
        errors before compensation when t is a multiple of the interval."""
        return self.reset_interval > 0 and t % self.reset_interval == 0

    @property
    def flags(self) -> int:
        return ob.ONEBIT_UNIT_SCALE if self.unit_scale else 0

    def compress(self, m: torch.Tensor, t: int, first: bool = False, stream=None) -> None:
        ob.onebit_compress_ex(m, self.ef, self.scales, self.bits, self.N, self.n, clip=self.clip,
                              reset=first or self.is_reset(t), seg_off=self.seg_off,
                              seg_k=self.seg_k, seg_err_ratio=self.seg_err_ratio,
                              n_seg=self.n_seg, flags=self.flags, ws=self.ws, stream=stream)

    def compress_grad(self, g: torch.Tensor, t: int, beta1: float, first: bool = False,
                      stream=None) -> None:
        """Compress from gradients: each worker's momentum is formed from g and
        the previous step's packed global momentum (sv_bits, sv_scales)."""
        ob.onebit_compress_ex(g, self.ef, self.scales, self.bits, self.N, self.n,
                              mb_bits=self.sv_bits, mb_scales=self.sv_scales, beta1=beta1,
                              clip=self.clip, reset=first or self.is_reset(t),
                              seg_off=self.seg_off, seg_k=self.seg_k,
                              seg_err_ratio=self.seg_err_ratio, n_seg=self.n_seg,
                              flags=self.flags, ws=self.ws, stream=stream)

    def server(self, t: int, first: bool = False, decompress: bool = True, stream=None) -> None:
        flags = self.flags
        sv_scales = self.sv_scales
        if self.keep_prev:  # this step's words go to the older buffer
            self.sv_bits, self.sv_bits_prev = self.sv_bits_prev, self.sv_bits
            flags |= ob.ONEBIT_KEEP_PREV
            sv_scales = self._sv_scales2
        ob.onebit_server_reduce_ex(self.bits, self.scales, self.sv_ef, sv_scales,
                                   self.sv_bits, self.mbar if decompress else None, self.N,
                                   self.n, reset=first or self.is_reset(t),
                                   seg_off=self.seg_off, seg_k=self.seg_k,
                                   seg_err_ratio=self.seg_err_ratio, n_seg=self.n_seg,
                                   flags=flags, ws=self.ws, stream=stream)

    # buffers that carry over from one step to the next (the worker sign words
    # and the workspace are rewritten by every step)
    _STATE = ("ef", "scales", "sv_ef", "sv_scales", "sv_bits", "mbar")

    _PREV = ("sv_bits_prev", "sv_scales_prev")

    def _state_names(self):
        return self._STATE + (self._PREV if self.keep_prev else ())

    def config(self) -> dict:
        return {"N": self.N, "n": self.n, "clip": self.clip,
                "reset_interval": self.reset_interval, "unit_scale": self.unit_scale,
                "keep_prev": self.keep_prev}

    def state_dict(self) -> Dict[str, Optional[torch.Tensor]]:
        """The group's carried state and its layer tables (None where unset),
        for ``checkpoint.save``."""
        d = {k: getattr(self, k) for k in self._state_names()}
        d.update(seg_off=self.seg_off, seg_k=self.seg_k, seg_err_ratio=self.seg_err_ratio)
        return d

    @classmethod
    def from_state(cls, tensors: Mapping[str, torch.Tensor], config: dict,
                   device) -> "OneBitGroup":
        """A group rebuilt from ``state_dict`` tensors and ``config()``."""
        grp = cls(int(config["N"]), int(config["n"]), device, clip=float(config["clip"]),
                  reset_interval=int(config["reset_interval"]),
                  seg_off=tensors.get("seg_off"), seg_k=tensors.get("seg_k"),
                  unit_scale=bool(config["unit_scale"]),
                  seg_err_ratio=tensors.get("seg_err_ratio"),
                  keep_prev=bool(config.get("keep_prev", False)))
        for k in grp._state_names():
            dst, src = getattr(grp, k), tensors[k]
            if dst.shape != src.shape or dst.dtype != src.dtype:
                raise ValueError(f"{k}: expected {tuple(dst.shape)} {dst.dtype}, "
                                 f"got {tuple(src.shape)} {src.dtype}")
            dst.copy_(src)
        return grp

    def worker_error(self) -> torch.Tensor:
        e = torch.empty_like(self.ef)
        ob.onebit_error_materialize(self.ef, self.scales, e, self.N, self.n, self.n)
        return e

    def server_error(self) -> torch.Tensor:
        e = torch.empty_like(self.sv_ef)
        ob.onebit_error_materialize(self.sv_ef, self.sv_scales, e, self.N, 1, self.n)
        return e

    def adam_step(self, x: torch.Tensor, v: torch.Tensor, lr: float, eps: float, stream=None) -> None:
        ob.frozen_v_step(mode=0, N=self.N, x=x, m=self.mbar, v=v, lr=lr, eps=eps, stream=stream)

    def capture_step(self, m: torch.Tensor, x: torch.Tensor, v: torch.Tensor, lr: float,
                     eps: float) -> "torch.cuda.CUDAGraph":
        """A HIP graph of one compressed Adam step that does not reset the
        errors: compress ``m``, server, and the decompression inside the Adam
        pass (x updated, the decompressed momentum in ``mbar``), on these fixed
        buffers.  Write the next momenta into ``m`` and replay it; the first
        step and every ``reset_interval``-th step reset the errors and run
        eagerly.  Nothing in the step allocates, clears memory or
        synchronises, so the graph holds only the library's kernels."""
        if self.keep_prev:
            raise ValueError("capture_step needs fixed server buffers (keep_prev=False)")
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(device=self.device)  # default priority
        side.wait_stream(torch.cuda.current_stream(self.device))
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                ob.onebit_compress_ex(m, self.ef, self.scales, self.bits, self.N, self.n,
                                      clip=self.clip, reset=False, seg_off=self.seg_off,
                                      seg_k=self.seg_k, seg_err_ratio=self.seg_err_ratio,
                                      n_seg=self.n_seg, flags=self.flags, ws=self.ws)
                ob.onebit_server_reduce_ex(self.bits, self.scales, self.sv_ef, self.sv_scales,
                                           self.sv_bits, None, self.N, self.n, reset=False,
                                           seg_off=self.seg_off, seg_k=self.seg_k,
                                           seg_err_ratio=self.seg_err_ratio, n_seg=self.n_seg,
                                           flags=self.flags, ws=self.ws)
                ob.frozen_v_step(mode=2, N=self.N, x=x, m=None, v=v, lr=lr, eps=eps,
                                 m_bits=self.sv_bits, m_scales=self.sv_scales, m_chunks=self.n,
                                 m_out=self.mbar)
        torch.cuda.current_stream(self.device).wait_stream(side)
        return graph

    def adam_step_packed(self, x: torch.Tensor, v: torch.Tensor, lr: float, eps: float,
                         decompress: bool = False, stream=None) -> None:
        """Adam step reading the global momentum packed (server words and
        scales); with ``decompress`` the same pass also writes the
        decompressed momentum to ``mbar``."""
        ob.frozen_v_step(mode=2, N=self.N, x=x, m=None, v=v, lr=lr, eps=eps, m_bits=self.sv_bits,
                         m_scales=self.sv_scales, m_chunks=self.n,
                         m_out=self.mbar if decompress else None, stream=stream)


@dataclass
class LambState:
    """Per-layer 1-bit LAMB state (1-bit LAMB page, algorithm paragraph)."""

    x: torch.Tensor          # [N] parameters
    v_frozen: torch.Tensor   # [N] v_Tw
    v_fresh: torch.Tensor    # [N] v_t
    m_prev: torch.Tensor     # [N] previous global momentum
    seg_off: torch.Tensor    # int64 [S+1]
    c_avg: torch.Tensor      # [S]
    r: torch.Tensor          # [S] r_{t-1} -> r_t
    c: torch.Tensor          # [S] c_{t-1} -> c_t
    ratio_max: torch.Tensor  # [S]
    err_ratio: torch.Tensor  # [S] c_{t-1} / c_t, for the next step's error feedback
    ws: torch.Tensor
    m_next: Optional[torch.Tensor] = None  # [N] spare buffer of step_packed

    @classmethod
    def create(cls, x, v_frozen, m_prev, seg_off, c_avg) -> "LambState":
        S = seg_off.numel() - 1
        dev = x.device
        return cls(x=x, v_frozen=v_frozen, v_fresh=v_frozen.clone(), m_prev=m_prev,
                   seg_off=seg_off, c_avg=c_avg, r=torch.ones(S, dtype=torch.float32, device=dev),
                   c=c_avg.clone(), ratio_max=torch.empty(S, dtype=torch.float32, device=dev),
                   err_ratio=torch.ones(S, dtype=torch.float32, device=dev),
                   ws=torch.empty(max(256, ob.frozen_v_workspace_bytes(x.numel(), S)),
                                  dtype=torch.uint8, device=dev))

    _STATE = ("x", "v_frozen", "v_fresh", "m_prev", "seg_off", "c_avg", "r", "c", "err_ratio")

    def state_dict(self) -> Dict[str, torch.Tensor]:
        return {k: getattr(self, k) for k in self._STATE}

    @classmethod
    def from_state(cls, tensors: Mapping[str, torch.Tensor]) -> "LambState":
        st = cls.create(tensors["x"], tensors["v_frozen"], tensors["m_prev"], tensors["seg_off"],
                        tensors["c_avg"])
        for k in ("v_fresh", "r", "c", "err_ratio"):
            getattr(st, k).copy_(tensors[k])
        return st

    def step(self, mbar: torch.Tensor, lr: float, eps: float, beta1: float, beta2: float,
             thr: float, r_min: float, r_max: float, use_c_t: bool = False, stream=None) -> None:
        """LAMB step on the decompressed global momentum ``mbar`` (m_t) with
        ``m_prev`` as m_{t-1}.  ``m_prev`` is the caller's: before the next
        step put m_t into it (``st.m_prev.copy_(mbar)``), since the server
        rewrites its own ``mbar`` on the next step; ``step_packed`` keeps it
        by itself."""
        S = self.seg_off.numel() - 1
        ob.frozen_v_step(mode=1, N=self.x.numel(), x=self.x, m=mbar, v=self.v_frozen, lr=lr,
                         eps=eps, beta1=beta1, beta2=beta2, m_prev=self.m_prev,
                         v_fresh=self.v_fresh, seg_off=self.seg_off, n_seg=S, c_avg=self.c_avg,
                         r_prev=self.r, c_prev=self.c, ratio_max=self.ratio_max,
                         r_threshold=thr, r_min=r_min, r_max=r_max, use_c_t=use_c_t,
                         err_ratio=self.err_ratio, ws=self.ws, stream=stream)

    def step_packed(self, bits: torch.Tensor, scales: torch.Tensor, seg_k: torch.Tensor,
                    chunks: int, lr: float, eps: float, beta1: float, beta2: float, thr: float,
                    r_min: float, r_max: float, use_c_t: bool = False,
                    prev_bits: Optional[torch.Tensor] = None,
                    prev_scales: Optional[torch.Tensor] = None,
                    stream=None) -> Optional[torch.Tensor]:
        """LAMB step reading the global momentum as the server's sign words and
        chunk scales, divided by the layer coefficients in the same pass.  The
        decompressed momentum it writes becomes ``m_prev`` for the next step
        and is returned.

        With ``prev_bits`` and ``prev_scales`` (the previous step's server
        words and scales, e.g. a ``keep_prev`` group's ``sv_bits_prev`` and
        ``sv_scales_prev``) m_{t-1} is decoded from them instead of read from
        ``m_prev``, and no decompressed momentum is written (unless
        ``use_c_t``, whose second pass reads it): ``m_prev`` is then left
        as it was and None is returned."""
        S = self.seg_off.numel() - 1
        prev = prev_bits is not None
        write_m = use_c_t or not prev
        if write_m and self.m_next is None:
            self.m_next = torch.empty_like(self.x)
        ob.frozen_v_step(mode=3, N=self.x.numel(), x=self.x, m=None, v=self.v_frozen, lr=lr,
                         eps=eps, beta1=beta1, beta2=beta2, m_prev=None if prev else self.m_prev,
                         v_fresh=self.v_fresh, seg_off=self.seg_off, n_seg=S, c_avg=self.c_avg,
                         r_prev=self.r, c_prev=self.c, ratio_max=self.ratio_max,
                         r_threshold=thr, r_min=r_min, r_max=r_max, use_c_t=use_c_t,
                         err_ratio=self.err_ratio, m_bits=bits, m_scales=scales, m_chunks=chunks,
                         m_seg_k=seg_k, m_out=self.m_next if write_m else None,
                         mp_bits=prev_bits, mp_scales=prev_scales, ws=self.ws, stream=stream)
        if not write_m:
            return None
        self.m_prev, self.m_next = self.m_next, self.m_prev
        return self.m_prev


@dataclass
class AdamWarmup:
    """Uncompressed Adam steps before the compressed phase (1-bit Adam
    article, section 2.1 and its warmup setting); ``v`` at the end is the
    frozen variance v_Tw of the compressed steps."""

    x: torch.Tensor  # [N] parameters
    m: torch.Tensor  # [N] momentum
    v: torch.Tensor  # [N] variance

    @classmethod
    def create(cls, x: torch.Tensor) -> "AdamWarmup":
        return cls(x=x, m=torch.zeros_like(x), v=torch.zeros_like(x))

    def state_dict(self) -> Dict[str, torch.Tensor]:
        return {"x": self.x, "m": self.m, "v": self.v}

    @classmethod
    def from_state(cls, tensors: Mapping[str, torch.Tensor]) -> "AdamWarmup":
        return cls(x=tensors["x"], m=tensors["m"], v=tensors["v"])

    def step(self, g: torch.Tensor, lr: float, eps: float, beta1: float, beta2: float,
             stream=None) -> None:
        """One step on the gradient averaged over the data-parallel group."""
        ob.warmup_adam_step(self.x, self.m, self.v, g, self.x.numel(), lr, eps, beta1, beta2,
                            stream=stream)


@dataclass
class LambWarmup:
    """Uncompressed LAMB steps before the compressed phase, and what they hand
    over (1-bit LAMB page): v_Tw, the coefficient average c_avg and the
    per-layer momentum scale k_l."""

    x: torch.Tensor        # [N] parameters
    m: torch.Tensor        # [N] momentum
    v: torch.Tensor        # [N] variance
    seg_off: torch.Tensor  # int64 [S+1]
    c: torch.Tensor        # [S] coefficients of the last step
    c_avg: torch.Tensor    # [S] their moving average
    ws: torch.Tensor
    steps: int = 0

    @classmethod
    def create(cls, x: torch.Tensor, seg_off: torch.Tensor) -> "LambWarmup":
        S = seg_off.numel() - 1
        dev = x.device
        return cls(x=x, m=torch.zeros_like(x), v=torch.zeros_like(x), seg_off=seg_off,
                   c=torch.ones(S, dtype=torch.float32, device=dev),
                   c_avg=torch.ones(S, dtype=torch.float32, device=dev),
                   ws=torch.empty(max(256, ob.warmup_workspace_bytes(x.numel(), S)),
                                  dtype=torch.uint8, device=dev))

    def state_dict(self) -> Dict[str, torch.Tensor]:
        """Carried tensors; the step count goes with the checkpoint's meta."""
        return {"x": self.x, "m": self.m, "v": self.v, "seg_off": self.seg_off, "c": self.c,
                "c_avg": self.c_avg}

    @classmethod
    def from_state(cls, tensors: Mapping[str, torch.Tensor], steps: int) -> "LambWarmup":
        lw = cls.create(tensors["x"], tensors["seg_off"])
        lw.m, lw.v = tensors["m"], tensors["v"]
        lw.c.copy_(tensors["c"])
        lw.c_avg.copy_(tensors["c_avg"])
        lw.steps = int(steps)
        return lw

    def step(self, g: torch.Tensor, lr: float, eps: float, beta1: float, beta2: float,
             beta_c: float, stream=None) -> None:
        """One step on the averaged gradient; the first starts the average."""
        ob.warmup_lamb_step(self.x, self.m, self.v, g, self.x.numel(), self.seg_off,
                            self.seg_off.numel() - 1, lr, eps, beta1, beta2, beta_c,
                            self.steps == 0, self.c, self.c_avg, self.ws, stream=stream)
        self.steps += 1

    def momentum_scale(self, stream=None) -> torch.Tensor:
        """k_l from the momentum at the end of warmup."""
        S = self.seg_off.numel() - 1
        k = torch.empty(S, dtype=torch.float32, device=self.x.device)
        ob.lamb_momentum_scale(self.m, self.x.numel(), self.seg_off, S, k, self.ws, stream=stream)
        return k

    def to_compressed(self) -> LambState:
        """The compressed phase's state: v_Tw = v, r = 1, c = c_avg, fresh
        variance v_Tw, previous global momentum m_Tw."""
        return LambState.create(self.x, self.v, self.m.clone(), self.seg_off, self.c_avg.clone())


def momentum_scale(m: torch.Tensor, seg_off: torch.Tensor, stream=None) -> torch.Tensor:
    """k_l of every layer from a momentum buffer m [N] (the end of warmup):
    ``lamb_momentum_scale`` with a workspace of its own."""
    N, S = m.numel(), seg_off.numel() - 1
    ws = torch.empty(max(256, ob.warmup_workspace_bytes(N, S)), dtype=torch.uint8,
                     device=m.device)
    k = torch.empty(S, dtype=torch.float32, device=m.device)
    ob.lamb_momentum_scale(m, N, seg_off, S, k, ws, stream=stream)
    return k
