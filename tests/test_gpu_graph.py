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


def test_next_rows_replay_in_a_graph(bsa):
    """Token permutation, estimator, forward with block mass, mask narrowing,
    a forward on the narrowed mask, the inverse permutation of O and a
    structured mask, captured once and replayed like the step above."""
    B, H, N, D, bs, p = 1, 4, 2900, 64, 128, 0.9
    q0, k0, v0, _ = _data(2, B, H, N, D)
    dev = q0.device
    R = bsa.num_rows(q0, bs)
    nb = -(-N // bs)
    cap = R * nb
    shape = bsa.make_shape(B, H, N, D, bs, 0)
    perm = torch.from_numpy(np.random.default_rng(3).permutation(N).astype(np.int32)).to(dev)
    from block_sparse_attention_16_amd import _lib as L
    kinds = torch.tensor([L.BSA_PATTERN_SPATIAL, L.BSA_PATTERN_TEMPORAL, L.BSA_PATTERN_DIAGONAL,
                          L.BSA_PATTERN_MULTI_DIAGONAL], dtype=torch.int32, device=dev)

    def csr():
        return bsa.Csr(torch.empty(R + 1, dtype=torch.int32, device=dev),
                       torch.empty(cap, dtype=torch.int32, device=dev))
    mask, narrow, smask = csr(), csr(), csr()
    ws_e = torch.empty(bsa.bsa_workspace_size(shape, 0, 0), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(bsa.bsa_workspace_size(shape, 1, cap), dtype=torch.uint8, device=dev)
    ws_s = torch.empty(bsa.bsa_workspace_size(shape, 3, 0), dtype=torch.uint8, device=dev)
    ws_p = torch.empty(bsa.bsa_workspace_size(shape, 4, 0), dtype=torch.uint8, device=dev)
    q, k, v, o, o2, o_back = (torch.empty_like(q0) for _ in range(6))
    lse, lse2 = (torch.empty((B, H, N), dtype=torch.float32, device=dev) for _ in range(2))
    mass, mass2 = (torch.empty(cap, dtype=torch.float32, device=dev) for _ in range(2))

    def step():
        for src, dst in ((q0, q), (k0, k), (v0, v)):
            bsa.bsa_permute_tokens(src, perm, out=dst)
        bsa.bsa_estimate_mask(q, k, p, bs, keep_prefix_tokens=130, out=mask, workspace=ws_e)
        bsa.bsa_forward(q, k, v, mask, bs, out=o, lse=lse, mass=mass, workspace=ws_f)
        bsa.bsa_select_from_mass(q, mask, mass, 0.8, bs, keep_prefix_tokens=130, out=narrow, workspace=ws_s)
        bsa.bsa_forward(q, k, v, narrow, bs, out=o2, lse=lse2, mass=mass2, workspace=ws_f)
        bsa.bsa_permute_tokens(o2, perm, inverse=True, out=o_back)
        bsa.bsa_structured_mask(q, kinds, bs, prefix_tokens=100, frame_tokens=640, band=2, period=5, out=smask,
                                workspace=ws_p)

    def snapshot():
        torch.cuda.synchronize()
        out = []
        for m in (mask, narrow, smask):
            rp = m.row_ptr.clone()
            out += [rp, m.col_idx[:int(rp[-1].item())].clone()]
        n1, n2 = int(mask.row_ptr[-1].item()), int(narrow.row_ptr[-1].item())
        return out + [q.clone(), o.clone(), lse.clone(), mass[:n1].clone(), o2.clone(), lse2.clone(),
                      mass2[:n2].clone(), o_back.clone()]

    def same(a, b):
        return all(x.shape == y.shape and torch.equal(x.view(torch.uint8) if x.dtype != torch.int32 else x,
                                                      y.view(torch.uint8) if y.dtype != torch.int32 else y)
                   for x, y in zip(a, b))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    ref = snapshot()
    assert int(narrow.row_ptr[-1].item()) < int(mask.row_ptr[-1].item())   # narrowing dropped entries

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in (mask.row_ptr, mask.col_idx, narrow.row_ptr, narrow.col_idx, smask.row_ptr, smask.col_idx, q, o,
                  lse, mass, o2, lse2, mass2, o_back):
            t.zero_()
        graph.replay()
        assert same(snapshot(), ref), f"replay {rep} differs from the eager step"
        bsa.bsa_permute_tokens(o, perm, inverse=True, out=torch.empty_like(o))   # eager work between replays
        torch.cuda.synchronize()
