"""The hot path under HIP graph capture (torch.cuda.CUDAGraph): estimator,
forward and backward captured once into preallocated buffers, replayed
several times with eager work and synchronisations between the replays;
every replay matches the eager result bit for bit, also after the inputs
change in place.  The library enqueues kernels only (no memset, copy or
allocation), so a caller's serving loop can capture it."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from tests.gpu_helpers import to_device
from workloads import round_to_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_16_amd as m
    m.load()
    return m


def _data(seed, B, H, N, D):
    rng = np.random.default_rng(seed)
    q = round_to_bf16(rng.normal(size=(B, H, N, D)).astype(np.float32) * 0.5)
    k = round_to_bf16(rng.normal(size=(B, H, N, D)).astype(np.float32) + q)
    v = round_to_bf16(rng.normal(size=(B, H, N, D)).astype(np.float32))
    g = round_to_bf16(rng.normal(size=(B, H, N, D)).astype(np.float32))
    return [to_device(t, "bf16") for t in (q, k, v, g)]


def test_estimate_forward_backward_replay_in_a_graph(bsa):
    B, H, N, D, bs, p = 1, 4, 3000, 128, 64, 0.9
    q, k, v, g = _data(0, B, H, N, D)
    R = bsa.num_rows(q, bs)
    nb = -(-N // bs)
    cap = R * nb
    dev = q.device
    shape = bsa.make_shape(B, H, N, D, bs, 0)
    mask = bsa.Csr(torch.empty(R + 1, dtype=torch.int32, device=dev), torch.empty(cap, dtype=torch.int32,
                                                                                   device=dev))
    ws_e = torch.empty(bsa.bsa_workspace_size(shape, 0, 0), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(bsa.bsa_workspace_size(shape, 1, cap), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(bsa.bsa_workspace_size(shape, 2, cap), dtype=torch.uint8, device=dev)
    o, o32, dq, dk, dv = (torch.empty_like(q), torch.empty(q.shape, dtype=torch.float32, device=dev),
                          torch.empty_like(q), torch.empty_like(q), torch.empty_like(q))
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    mass = torch.empty(cap, dtype=torch.float32, device=dev)

    def step():
        bsa.bsa_estimate_mask(q, k, p, bs, out=mask, workspace=ws_e)
        bsa.bsa_forward(q, k, v, mask, bs, out=o, lse=lse, mass=mass, workspace=ws_f, o32=o32)
        bsa.bsa_backward(q, k, v, o, g, lse, mask, bs, workspace=ws_b, dq=dq, dk=dk, dv=dv, o32=o32)

    def snapshot():
        torch.cuda.synchronize()
        rp = mask.row_ptr.clone()
        n = int(rp[-1].item())
        return [rp, mask.col_idx[:n].clone(), o.clone(), lse.clone(), mass[:n].clone(), dq.clone(), dk.clone(),
                dv.clone()]

    def same(a, b):
        return all(x.shape == y.shape and torch.equal(x.view(torch.uint8) if x.dtype != torch.int32 else x,
                                                      y.view(torch.uint8) if y.dtype != torch.int32 else y)
                   for x, y in zip(a, b))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # warm-up on the capturing side stream
    torch.cuda.current_stream().wait_stream(side)
    ref = snapshot()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    other = torch.zeros_like(o)
    for rep in range(3):
        for t in (mask.row_ptr, mask.col_idx, o, lse, mass, dq, dk, dv):
            t.zero_()
        graph.replay()
        got = snapshot()
        assert same(got, ref), f"replay {rep} differs from the eager step"
        bsa.bsa_forward(q, k, v, mask, bs, out=other, want_mass=False)   # eager work between replays
        torch.cuda.synchronize()

    # new inputs in place: the replay reads them
    q2, k2, v2, g2 = _data(1, B, H, N, D)
    for dst, src in ((q, q2), (k, k2), (v, v2), (g, g2)):
        dst.copy_(src)
    step()
    ref2 = snapshot()
    assert not same(ref2, ref)
    graph.replay()
    assert same(snapshot(), ref2), "replay after an input change differs from the eager step"
