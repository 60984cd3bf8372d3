"""The blocked pass under HIP graph capture (needs an MI355X).

A caller may capture dbs_smooth into a graph: the library's second stream
joins the capture through its ordering events, so the graph holds both
streams' launches and their dependencies.  Each case captures one pass, then
replays the graph three times with eager work in between, and checks every
replay against the oracle bit for bit.
"""
import numpy as np
import pytest
import torch

import distance_geometry_bound_amd as dgb
import oracle
from distance_geometry_bound_amd import gen

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


# (130, 129): at the automatic choice the lead schedule on one stream; with
# lead=False a batch split over the two streams
@pytest.mark.parametrize("n,batch,bands,blocks,lead", [
    (700, 1, 2, 2, None), (700, 1, 2, 4, None), (385, 2, 1, 1, None), (385, 2, 0, 2, None),
    (130, 129, -1, -1, None), (130, 129, -1, -1, False), (385, 2, 0, 1, True)])
def test_captured_pass_replays_match_oracle(n, batch, bands, blocks, lead):
    U0, L0, _ = gen.random_sound_bounds(n, seed=500 + n + bands, batch=batch, box=6.0 + n / 8)
    Ue, Le = oracle.smooth(U0, L0)
    Ui = torch.from_numpy(U0).to(DEV)
    Li = torch.from_numpy(L0).to(DEV)
    U, L = torch.empty_like(Ui), torch.empty_like(Li)
    kw = dict(algo="blocked", lookahead=None if bands < 0 else bands,
              step_blocks=None if blocks < 0 else blocks, lead=lead)
    s = torch.cuda.Stream(DEV)
    s.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(s):               # warm-up on the capture stream
        U.copy_(Ui)
        L.copy_(Li)
        dgb.smooth(U, L, **kw)
    torch.cuda.current_stream(DEV).wait_stream(s)
    torch.cuda.synchronize(DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        U.copy_(Ui)
        L.copy_(Li)
        dgb.smooth(U, L, **kw)
    torch.cuda.synchronize(DEV)
    for rep in range(3):
        U.fill_(-1.0)
        L.fill_(-1.0)
        g.replay()
        torch.cuda.synchronize(DEV)
        tag = f"n={n} batch={batch} bands={bands} blocks={blocks} replay {rep}"
        assert np.array_equal(U.cpu().numpy().view(np.uint32), Ue.view(np.uint32)), tag
        assert np.array_equal(L.cpu().numpy().view(np.uint32), Le.view(np.uint32)), tag
        # eager work between replays, on the same buffers and on the
        # capture stream, whose library stream is part of the graph
        U.copy_(Ui)
        L.copy_(Li)
        dgb.smooth(U, L, **kw)
        with torch.cuda.stream(s):
            U2, L2 = Ui.clone(), Li.clone()
            dgb.smooth(U2, L2, **kw)
        torch.cuda.synchronize(DEV)
        assert np.array_equal(U2.cpu().numpy().view(np.uint32), Ue.view(np.uint32)), tag
        assert np.array_equal(L2.cpu().numpy().view(np.uint32), Le.view(np.uint32)), tag
    del g
