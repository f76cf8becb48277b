"""The issue-rate probes (include/fa_probe.h) on the GPU: every wave reports,
where it ran is what the probes assume, and the rates are in a plausible
range (a v_mfma_f32_32x32x16_bf16 occupies its SIMD's matrix core for at
least 16 cycles; a wave issues at most one vector instruction per cycle)."""
import pytest

from exact_attention_16_amd import probe

pytestmark = pytest.mark.gpu


def test_mfma_alone():
    res = probe.run(probe.MFMA, 16, probe.NONE, 0, 1, repeats=1)
    assert len(res) == 4
    for cyc, simd, _ in res:
        assert 16 <= cyc / (16 * 16) <= 256
    res = probe.run(probe.MFMA_DEP, 16, probe.NONE, 0, 1, repeats=1)
    for cyc, simd, _ in res:
        assert 16 <= cyc / (16 * 16) <= 1024


def test_fma_two_waves_per_simd():
    res = probe.run(probe.FMA, 64, probe.FMA, 64, 2, repeats=1)
    assert len(res) == 8
    for cyc, _, _ in res:
        assert 1 <= cyc / (32 * 64) <= 256


def test_idle_slot_reports_zero_and_mix_runs():
    res = probe.run(probe.NONE, 0, probe.EXP, 16, 2, repeats=1)
    assert all(c == 0 for c, _, _ in res[:4])
    assert all(c > 0 for c, _, _ in res[4:])
    res = probe.run(probe.MIX, 4, probe.NONE, 0, 1, mix=8, repeats=1)
    assert all(c > 0 for c, _, _ in res)
