"""The matrix-core microbenchmarks (libsfa_probe.so) that bench.py reports the attention
kernel against: each probe runs, and its figures are self-consistent (needs an MI355X)."""
import sys

import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

PEAK = 2516.6   # MI355X dense bf16 MFMA, TFLOP/s


def test_probes_report_consistent_figures():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    from sparse_attention_frame_amd import probe

    got = {}
    for kind in (probe.MFMA_CHAIN, probe.TILE_LOOP, probe.TILE_LOOP64, probe.TILE_NOEXP):
        r = probe.run(kind, waves=8, iters=4000)
        print(f"[probe] kind {kind}: {r}", file=sys.stderr, flush=True)
        assert r["ms"] > 0 and 0.5 < r["clock_ghz"] < 2.6
        assert 0 < r["tflops"] < 1.02 * PEAK
        # busy = MFMA cycles / (time x clock): consistent with the rate and the clock
        assert abs(r["mfma_busy"] - r["tflops"] / PEAK * 2.4 / r["clock_ghz"]) < 0.02
        got[kind] = r["tflops"]
    # the loop with the softmax is slower than without it, and both below bare MFMA chains
    assert got[probe.TILE_LOOP] < got[probe.TILE_NOEXP] < got[probe.MFMA_CHAIN]
    r4 = probe.run(probe.MFMA_CHAIN, waves=4, iters=4000)
    assert r4["tflops"] > 0
    with pytest.raises(RuntimeError):
        probe.run(probe.MFMA_CHAIN, waves=6, iters=10)
