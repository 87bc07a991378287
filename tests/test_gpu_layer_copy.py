"""The layer-granular copy comparator: a layer whose 384 experts all sit in
pinned host memory is copied whole into HBM (by the gather kernel with every
expert picked, then by the DMA engines), every copied blob equals the host
bytes, and the layer computed on the copy equals the same layer fully
resident, bit for bit."""
import os
import sys

import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


@pytest.mark.timeout(300)
def test_layer_copy_comparator():
    r = bench.measure_layer_copy(T=8, layers=1, reps=1)
    assert r["blobs_compared"] == 384
    assert r["gather_copy_bit_exact"] and r["dma_copy_bit_exact"]
    assert r["forward_on_copy_equals_resident"]
