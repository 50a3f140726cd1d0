"""A HIP graph of the compressed Adam step (OneBitGroup.capture_step) replayed
for several steps, with eager work and synchronisations between the replays,
must give bit for bit what the same steps give when run eagerly."""

import numpy as np
import pytest
import torch

from momentum_compression_amd.state import OneBitGroup
from tests._gpu import device, gen, host

pytestmark = pytest.mark.gpu

STATE = ("ef", "scales", "sv_ef", "sv_scales", "sv_bits", "mbar")


def _same(a, b):
    return np.array_equal(host(a).view(np.uint8), host(b).view(np.uint8))


@pytest.mark.parametrize("n,L,clip", [(8, 3 * 1024 + 64, 0.0), (16, 1024, 2e-3), (5, 2368, 0.0)])
def test_graph_replays_match_eager(n, L, clip):
    dev = device()
    N = n * L
    print(f"[graph] N={N} n={n} clip={clip}", flush=True)
    gx = gen(11, dev)
    x0 = torch.randn(N, generator=gx, device=dev) * 0.02
    v = torch.rand(N, generator=gx, device=dev) * 1e-6 + 1e-8

    def momentum(t):
        return torch.randn((n, N), generator=gen(300 + t, dev), device=dev) * 1e-3

    eager = OneBitGroup(N, n, dev, clip=clip)
    xe = x0.clone()
    graphed = OneBitGroup(N, n, dev, clip=clip)
    xg = x0.clone()
    m_buf = torch.empty((n, N), device=dev)
    # the first step resets the errors: eager on both
    for grp, x in ((eager, xe), (graphed, xg)):
        grp.compress(momentum(1), 1, first=True)
        grp.server(1, first=True, decompress=False)
        grp.adam_step_packed(x, v, 1e-3, 1e-6, decompress=True)
    graph = graphed.capture_step(m_buf, xg, v, 1e-3, 1e-6)
    torch.cuda.synchronize()
    for t in range(2, 7):
        m = momentum(t)
        eager.compress(m, t)
        eager.server(t, decompress=False)
        eager.adam_step_packed(xe, v, 1e-3, 1e-6, decompress=True)
        torch.cuda.synchronize()          # eager work, then a synchronisation
        m_buf.copy_(m)
        graph.replay()
        torch.cuda.synchronize()
        assert _same(xe, xg), f"t={t} parameters"
        for name in STATE:
            assert _same(getattr(eager, name), getattr(graphed, name)), f"t={t} {name}"
