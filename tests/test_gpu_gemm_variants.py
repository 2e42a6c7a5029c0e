"""Every grouped-GEMM kernel variant, forced one at a time through
MOE_GEMM_CFG, against the oracle on whole layers (forward and backward, all
outputs element by element).  The default selection uses only some of the
variants at the benchmark shapes; this runs each on shapes every variant
accepts (128- and 256-divisible N, M and K), with ragged expert groups, and
in a second layer with a shared expert and sigmoid routing."""
import numpy as np
import pytest

from mixture_experts_layer_23_amd import synthetic as S
from tests.gpu_common import note
from tests.test_gpu_parity import compare_layer, oracle_layer, run_layer

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

# 0 register-staged; 1 128x128 DMA, 2 stages; 2 256x128 DMA, 3 stages;
# 3 / 4 256x256 / 256x128 on 4 waves; 5 / 6 the same on 8 waves;
# 7 / 8 persistent 256x256 / 256x128; 9 256x128 on 4 waves with 32-deep
# slabs, two workgroups per CU; 10 / 11 256x256 tile loop with the next
# tile's first slabs fetched during the epilogue, two 64-deep / four 32-deep
# stages (9-11 are weight-gradient kernels: the row GEMMs take 1)
CFGS = list(range(12))
WORKLOADS = {
    "minimind_like": S.WORKLOADS["minimind"].with_(T=512, D=512, F=512, E=4, K=2),
    "shared_sigmoid": S.WORKLOADS["deepseek_v3"].with_(T=384, D=512, F=512, E=8, K=2),
    # F = 576: reductions over F (and the gate / up split of the stacked
    # reduction at k = F) take an odd number of 64-deep slabs, so the
    # pipelines end on their other stage; the GEMMs whose N = F is not
    # 128-divisible run on the register-staged kernel
    "odd_reduction": S.WORKLOADS["minimind"].with_(T=512, D=512, F=576, E=4, K=2),
    # F = 640: the gate/up forward has 2F / 128 = 10 column tiles, so its
    # 2-D tile blocks per XCD split the columns in two (not four)
    "xcd_two_column_groups": S.WORKLOADS["minimind"].with_(T=512, D=512, F=640, E=4, K=2),
    # 64 routed experts (+ a shared one): the 256-row kernels give each XCD a
    # block of the real m-tiles in the plain-store row GEMMs
    "many_experts": S.WORKLOADS["deepseek_v3"].with_(T=512, D=1024, F=256, E=64, K=8),
    # 128 slots over 256 experts: most groups are empty, so the weight-gradient
    # tile loops run long runs of empty tiles (zero stores, then the next
    # tile's slabs issued by hand) between the shared expert's and the few
    # routed experts' tiles
    "mostly_empty": S.WORKLOADS["deepseek_v3"].with_(T=64, D=512, F=256, E=256, K=2),
}
_ref = {}


@pytest.fixture(scope="module", autouse=True)
def gpu_only():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("cfg", CFGS)
@pytest.mark.parametrize("name", list(WORKLOADS))
def test_gemm_variant_layer_parity(name, cfg, monkeypatch):
    wl = WORKLOADS[name]
    monkeypatch.setenv("MOE_GEMM_CFG", str(cfg))
    note(f"GEMM variant {cfg} on {name}: {wl}")
    hin, layer = run_layer(wl)
    if name not in _ref:
        _ref[name] = oracle_layer(wl, hin)
    compare_layer(wl, hin, layer, _ref[name])
