"""GPU parity of the forward's pair grid (64-token blocks, bf16): a workgroup
takes query blocks 2m and 2m + 1 of a head and walks the union of their key
lists when both are strictly ascending lists of valid ids, else the two rows
one after the other.  The oracle attends each row's entries as listed, so
every form a CSR row can take is checked against it: ascending rows, empty
rows, rows that repeat, reverse or shuffle ids, pairs with one ascending row,
an odd number of blocks (the last pair holds one row) and a ragged last
block.  Ids outside [0, nb) carry no keys: their rows are compared with the
oracle on the row without them, and their block mass must be 0."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import bsa_oracle as O
from workloads import round_to_bf16
from tests.gpu_helpers import assert_forward_within, compare_forward, default_scale, to_device, to_host

pytestmark = pytest.mark.gpu

BS = 64


@pytest.fixture(scope="module")
def bsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_16_amd as m
    m.load()
    return m


def _inputs(rng, B, H, N, D):
    q = round_to_bf16(0.5 * rng.normal(size=(B, H, N, D)).astype(np.float32))
    k = round_to_bf16(rng.normal(size=(B, H, N, D)).astype(np.float32))
    v = round_to_bf16(rng.normal(size=(B, H, N, D)).astype(np.float32))
    return q, k, v


def _rows(rng, B, H, nb):
    """Row forms by (query block + 3 head) mod 8: empty, ids repeated,
    descending, shuffled, and four strictly ascending forms, so that pairs mix
    ascending and non-ascending rows differently in every head."""
    rows = []
    for bh in range(B * H):
        for i in range(nb):
            c = np.sort(rng.choice(nb, size=int(rng.integers(1, nb + 1)), replace=False))
            kind = (i + 3 * bh) % 8
            if kind == 0:
                rows.append(np.zeros(0, np.int64))
            elif kind == 1:
                rows.append(np.repeat(c[:4], 2))
            elif kind == 2:
                rows.append(c[::-1].copy())
            elif kind == 3:
                rows.append(rng.permutation(c))
            else:
                rows.append(c)
    return rows


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("N", [7 * BS - 13, 8 * BS, 1])
def test_pair_grid_rows_as_listed(bsa, D, N):
    rng = np.random.default_rng(31 * N + D)
    B, H = 1, 3
    nb = O.num_blocks(N, BS)
    q, k, v = _inputs(rng, B, H, N, D)
    rp, ci = O.rows_to_csr(_rows(rng, B, H, nb))
    mask = bsa.csr_from_host(rp, ci, "cuda")
    qd, kd, vd = (to_device(t, "bf16") for t in (q, k, v))
    o32 = torch.empty(qd.shape, dtype=torch.float32, device="cuda")
    o, lse, mass = bsa.bsa_forward(qd, kd, vd, mask, BS, o32=o32)
    torch.cuda.synchronize()
    err = compare_forward(q, k, v, BS, rp, ci, default_scale(D), list(range(B * H * nb)), to_host(o),
                          to_host(lse), to_host(mass), "bf16", o32_gpu=o32.cpu().numpy())
    assert_forward_within(err, "bf16", f"pair grid N={N} D={D}")


@pytest.mark.parametrize("D", [64, 128])
def test_pair_grid_ids_outside_the_grid(bsa, D):
    rng = np.random.default_rng(5 + D)
    B, H, N = 1, 2, 9 * BS - 30
    nb = O.num_blocks(N, BS)
    q, k, v = _inputs(rng, B, H, N, D)
    rows, clean = [], []
    for r in range(B * H * nb):
        c = np.sort(rng.choice(nb, size=int(rng.integers(1, nb + 1)), replace=False))
        clean.append(c)
        if r % 3 == 1:                      # out-of-grid ids around and inside an ascending row
            c = np.concatenate([[-1], c[: c.size // 2], [nb, nb + 7], c[c.size // 2:], [-5]])
        rows.append(c)
    rp, ci = O.rows_to_csr(rows)
    mask = bsa.csr_from_host(rp, ci, "cuda")
    qd, kd, vd = (to_device(t, "bf16") for t in (q, k, v))
    o, lse, mass = bsa.bsa_forward(qd, kd, vd, mask, BS)
    torch.cuda.synchronize()
    mass = to_host(mass)
    crp, cci = O.rows_to_csr(clean)
    # O and LSE against the oracle on the rows without the out-of-grid ids
    err = compare_forward(q, k, v, BS, crp, cci, default_scale(D), list(range(B * H * nb)), to_host(o),
                          to_host(lse), None, "bf16")
    assert_forward_within(err, "bf16", f"out-of-grid ids D={D}")
    # block mass: 0 on out-of-grid entries, the oracle's on the others
    _, _, mo = O.sparse_forward(q, k, v, BS, crp, cci, default_scale(D))
    for r in range(B * H * nb):
        got = mass[rp[r]:rp[r + 1]]
        ids = ci[rp[r]:rp[r + 1]]
        ok = (ids >= 0) & (ids < nb)
        assert np.all(got[~ok] == 0.0), f"row {r}: out-of-grid entries carry mass"
        assert np.abs(got[ok] - mo[crp[r]:crp[r + 1]]).max() <= 1e-4, f"row {r}: block mass"


@pytest.mark.parametrize("D", [64, 128])
def test_pair_grid_rows_independent_bitwise(bsa, D):
    """A row's results do not depend on the other row of its pair: the units
    its row does not list add exact zeros and leave its running max alone.
    The forward over a mask whose odd rows are emptied gives the even rows,
    bit for bit, the values they get with their neighbours present."""
    rng = np.random.default_rng(77 + D)
    B, H, N = 1, 2, 12 * BS - 3
    nb = O.num_blocks(N, BS)
    q, k, v = _inputs(rng, B, H, N, D)
    full = [np.sort(rng.choice(nb, size=int(rng.integers(1, nb + 1)), replace=False)) for _ in range(B * H * nb)]
    alone = [row if (r % nb) % 2 == 0 else np.zeros(0, np.int64) for r, row in enumerate(full)]
    qd, kd, vd = (to_device(t, "bf16") for t in (q, k, v))
    outs = []
    for rows in (full, alone):
        rp, ci = O.rows_to_csr(rows)
        o, lse, mass = bsa.bsa_forward(qd, kd, vd, bsa.csr_from_host(rp, ci, "cuda"), BS)
        torch.cuda.synchronize()
        outs.append((rp, o.cpu(), lse.cpu(), mass.cpu()))
    (rp1, o1, l1, m1), (rp2, o2, l2, m2) = outs
    for r in range(B * H * nb):
        bh, i = divmod(r, nb)
        if i % 2:
            continue
        lo, hi = i * BS, min(i * BS + BS, N)
        assert torch.equal(o1[0, bh, lo:hi], o2[0, bh, lo:hi]), f"row {r}: O depends on the neighbour row"
        assert torch.equal(l1[0, bh, lo:hi], l2[0, bh, lo:hi]), f"row {r}: LSE depends on the neighbour row"
        assert torch.equal(m1[rp1[r]:rp1[r + 1]], m2[rp2[r]:rp2[r + 1]]), f"row {r}: block mass"


@pytest.mark.parametrize("D", [64, 128])
def test_pair_grid_entries_past_capacity(bsa, D):
    """A capacity that ends inside a row: that row keeps its entries below the
    capacity, later rows have none (their O is 0, their LSE -inf), as in the
    single-row grid of 128-token blocks."""
    rng = np.random.default_rng(13 + D)
    B, H, N = 1, 2, 11 * BS - 9
    nb = O.num_blocks(N, BS)
    q, k, v = _inputs(rng, B, H, N, D)
    rows = [np.sort(rng.choice(nb, size=int(rng.integers(2, nb + 1)), replace=False)) for _ in range(B * H * nb)]
    rp, ci = O.rows_to_csr(rows)
    cut = nb + 3                              # a row of the second head, counted from its first row
    cap = int(rp[cut] + (rp[cut + 1] - rp[cut]) // 2)
    mask = bsa.csr_from_host(rp, ci, "cuda", capacity=cap)
    qd, kd, vd = (to_device(t, "bf16") for t in (q, k, v))
    o, lse, mass = bsa.bsa_forward(qd, kd, vd, mask, BS)
    torch.cuda.synchronize()
    clipped = [ci[rp[r]:min(rp[r + 1], cap)] if rp[r] < cap else np.zeros(0, np.int64) for r in range(len(rows))]
    crp, cci = O.rows_to_csr(clipped)
    assert crp[-1] == cap
    err = compare_forward(q, k, v, BS, crp, cci, default_scale(D), list(range(B * H * nb)), to_host(o),
                          to_host(lse), to_host(mass)[:cap], "bf16")
    assert_forward_within(err, "bf16", f"capacity cut D={D}")


@pytest.mark.parametrize("D", [64, 128])
def test_pair_grid_mask_with_no_entries(bsa, D):
    """A mask with no entries at all (capacity 0): every query gets O = 0 and
    LSE = -inf, and the backward gives zero gradients."""
    rng = np.random.default_rng(3 + D)
    B, H, N = 1, 2, 5 * BS - 7
    nb = O.num_blocks(N, BS)
    q, k, v = _inputs(rng, B, H, N, D)
    rp = np.zeros(B * H * nb + 1, np.int64)
    mask = bsa.csr_from_host(rp, np.zeros(0, np.int64), "cuda")
    assert mask.capacity == 0
    qd, kd, vd = (to_device(t, "bf16") for t in (q, k, v))
    o32 = torch.empty(qd.shape, dtype=torch.float32, device="cuda")
    o, lse, _ = bsa.bsa_forward(qd, kd, vd, mask, BS, want_mass=False, o32=o32)
    g = to_device(round_to_bf16(rng.normal(size=(B, H, N, D)).astype(np.float32)), "bf16")
    dq, dk, dv = bsa.bsa_backward(qd, kd, vd, o, g, lse, mask, BS, o32=o32)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(o32 == 0)
    assert torch.all(torch.isneginf(lse))
    assert torch.all(dq == 0) and torch.all(dk == 0) and torch.all(dv == 0)
