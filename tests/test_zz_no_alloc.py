"""bsa_select_from_mass_noalloc (no workspace; the library's static per-GPU
scratch) against bsa_select_from_mass (caller workspace), called through the
C ABI: two calls in a row, the second on a smaller problem, each compared
bit for bit (row_ptr and every col_idx entry) with the workspace version on
the same inputs."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_16_amd as m
    return m, m._lib if hasattr(m, "_lib") else None


def _case(rng, H, nb, bs):
    R = H * nb
    rows = []
    for r in range(R):
        if r % 11 == 4:
            rows.append(np.zeros(0, np.int64))
        else:
            rows.append(np.sort(rng.choice(nb, size=int(rng.integers(1, nb + 1)), replace=False)))
    counts = np.array([x.size for x in rows])
    rp = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    ci = np.concatenate(rows).astype(np.int32)
    mass = rng.random(ci.size).astype(np.float32)
    mass[rng.random(ci.size) < 0.02] = 0.0
    return rp, ci, mass


def _call(L, fn, shape, rp_d, ci_d, mass_d, p, keep, R, cap, ws=None):
    from block_sparse_attention_16_amd import _lib
    out_rp = torch.full((R + 1,), -7, dtype=torch.int32, device="cuda")
    out_ci = torch.full((cap,), -7, dtype=torch.int32, device="cuda")
    mask = _lib.BsaCsr(rp_d.data_ptr(), ci_d.data_ptr(), ci_d.numel())
    out = _lib.BsaCsr(out_rp.data_ptr(), out_ci.data_ptr(), cap)
    stream = torch.cuda.current_stream().cuda_stream
    if ws is None:
        st = fn(ctypes.byref(shape), ctypes.byref(mask), mass_d.data_ptr(), p, keep, ctypes.byref(out), stream)
    else:
        st = fn(ctypes.byref(shape), ctypes.byref(mask), mass_d.data_ptr(), p, keep, ctypes.byref(out),
                ws.data_ptr(), ws.numel(), stream)
    assert st == 0, L.bsa_last_error()
    torch.cuda.synchronize()
    n = int(out_rp[-1].item())
    return out_rp.cpu().numpy(), out_ci[:n].cpu().numpy()


def test_noalloc_narrowing_matches_workspace_version(lib):
    from block_sparse_attention_16_amd import _lib
    L = _lib.load()
    rng = np.random.default_rng(2024)
    # first call: 6 heads x 300 blocks; second call: smaller, 2 heads x 70 blocks
    for H, nb, bs, p, keep in ((6, 300, 128, 0.85, 130), (2, 70, 64, 0.6, 0)):
        N = nb * bs - 17
        rp, ci, mass = _case(rng, H, nb, bs)
        R, cap = H * nb, H * nb * nb
        shape = _lib.BsaShape(1, H, N, 64, bs, _lib.BSA_BF16)
        rp_d = torch.from_numpy(rp).cuda()
        ci_d = torch.from_numpy(ci).cuda()
        mass_d = torch.from_numpy(mass).cuda()
        ws = torch.empty(L.bsa_workspace_size(ctypes.byref(shape), _lib.BSA_WS_SELECT_FROM_MASS, 0),
                         dtype=torch.uint8, device="cuda")
        pf = float(np.float32(p))
        want_rp, want_ci = _call(L, L.bsa_select_from_mass, shape, rp_d, ci_d, mass_d, pf, keep, R, cap, ws=ws)
        got_rp, got_ci = _call(L, L.bsa_select_from_mass_noalloc, shape, rp_d, ci_d, mass_d, pf, keep, R, cap)
        assert np.array_equal(got_rp, want_rp), (H, nb)
        assert np.array_equal(got_ci, want_ci), (H, nb)
        assert 0 < got_rp[-1] < rp[-1] + R       # narrowed, plus forced blocks at most
