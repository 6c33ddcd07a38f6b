"""The measured matrix-core ceiling reported beside the published peak (needs an MI355X).

flide_measure_mfma_peak times a loop of independent bf16 16x16x32 products; the figure must be positive and
below the published dense bf16 peak of MI355X (2.5 PFLOP/s), and a bad argument must be rejected before
anything is launched.
"""
import pytest

pytestmark = pytest.mark.gpu


def test_measured_mfma_peak_is_below_the_published_peak():
    import torch
    from tree_forked_hybrid_amd import flide as F
    assert torch.cuda.is_available()
    v = F.flide_measure_mfma_peak(512, torch.cuda.current_stream())
    assert 100.0 < v < 2500.0, v


def test_measured_mfma_peak_rejects_bad_arguments():
    from tree_forked_hybrid_amd import flide as F
    with pytest.raises(F.FlideError):
        F.flide_measure_mfma_peak(0)
