"""flashtopk_probe_mfma: the matrix-core throughput kernel runs and reports a
rate of the right order for each instruction (MI355X only).  The bounds are
loose: the published dense peaks (FP8 5.0, BF16 2.5 PFLOP/s at 2.4 GHz) cap
it, and a quarter of them is far below any healthy reading."""
import pytest

import sparse_attention_indexer_fp8_amd as ftk

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,peak", [(ftk.FLASHTOPK_FP8_E4M3, 5033.0), (ftk.FLASHTOPK_BF16, 2517.0)],
                         ids=["fp8", "bf16"])
def test_probe_rate_is_plausible(dtype, peak):
    tf = ftk.flashtopk_probe_mfma(dtype, 20000)
    print("probe", dtype, round(tf, 1), "TFLOP/s", flush=True)
    assert 0.25 * peak < tf < 1.02 * peak


def test_probe_rejects_bad_arguments():
    with pytest.raises(ftk.FlashTopKError):
        ftk.flashtopk_probe_mfma(5, 10)
    with pytest.raises(ftk.FlashTopKError):
        ftk.flashtopk_probe_mfma(ftk.FLASHTOPK_FP8_E4M3, 0)
