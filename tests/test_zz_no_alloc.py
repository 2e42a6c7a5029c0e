"""moe_permute_noalloc (the permute without a workspace argument, for callers
that cannot allocate) against moe_permute through the C ABI: every output bit
for bit, on two calls in a row, the second with a smaller input, both on the
tiled path that uses the static scratch array; then a call on the
one-workgroup path (no scratch) for completeness."""
import numpy as np
import pytest

from mixture_experts_layer_23_amd import _lib as L
from tests.gpu_common import note, to_host

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu_only():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.lib()


def top_k(T, E, K, seed):
    """distinct experts per token from seeded random keys (skewed loads)"""
    rng = np.random.default_rng(seed)
    keys = rng.standard_normal((T, E)) + np.linspace(1.5, 0.0, E)[None, :]
    return np.argsort(-keys, axis=1, kind="stable")[:, :K].astype(np.int32)


def outputs(spec_cfg, T, E, K, D, rows):
    dev = "cuda"
    z = lambda n: torch.full((n,), -7, dtype=torch.int32, device=dev)
    return dict(counts=z(E), offsets=z(spec_cfg["G"] + 1), slot_row=z(T * K),
                row_token=z(rows), row_slot=z(rows), n_dropped=z(4),
                x_perm=torch.zeros(rows, D, dtype=torch.bfloat16, device=dev))


CASES = [  # (T, E, K, local range, shared, capacity factor): tiled path, then smaller
    (8192, 64, 8, (0, 32), 1, 1.0),
    (5000, 64, 8, (8, 40), 0, 0.0),
    (1000, 16, 4, (0, 16), 1, 1.25),  # one-workgroup path (no scratch)
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_permute_noalloc_matches_permute(case):
    T, E, K, (lo, hi), S, cap = CASES[case]
    D = 256
    note(f"permute_noalloc T={T} E={E} K={K} local=[{lo},{hi}) shared={S} cap={cap}")
    cfg = L.make_config(T, D, E, K, 256, lo, hi, S, L.MOE_SCORE_SOFTMAX, L.MOE_GATE_RENORM,
                        L.MOE_BF16, cap)
    rows = L.rows_max(cfg)
    idx = torch.from_numpy(top_k(T, E, K, seed=case)).cuda()
    x = torch.randn(T, D, device="cuda").to(torch.bfloat16)
    ws = torch.empty(max(L.workspace_size(cfg), 256), dtype=torch.uint8, device="cuda")
    G = hi - lo + S
    a = outputs(dict(G=G), T, E, K, D, rows)
    b = outputs(dict(G=G), T, E, K, D, rows)
    L.moe_permute(cfg, idx, x, a["counts"], a["offsets"], a["slot_row"], a["row_token"],
                  a["row_slot"], a["n_dropped"], a["x_perm"], ws)
    L.moe_permute_noalloc(cfg, idx, x, b["counts"], b["offsets"], b["slot_row"], b["row_token"],
                          b["row_slot"], b["n_dropped"], b["x_perm"])
    torch.cuda.synchronize()
    n = int(to_host(a["offsets"])[G])
    for k in ("counts", "offsets", "slot_row", "n_dropped"):
        np.testing.assert_array_equal(to_host(b[k]), to_host(a[k]), err_msg=k)
    for k in ("row_token", "row_slot"):
        np.testing.assert_array_equal(to_host(b[k])[:n], to_host(a[k])[:n], err_msg=k)
    r = int(to_host(a["offsets"])[hi - lo])  # routed rows (the shared rows are not gathered)
    np.testing.assert_array_equal(to_host(b["x_perm"])[:r], to_host(a["x_perm"])[:r])
    note(f"  rows {n}, dropped {int(to_host(a['n_dropped'])[0])}: bit-identical")
