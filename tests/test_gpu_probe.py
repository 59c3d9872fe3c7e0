"""GPU: the issue-rate diagnostics (attn_probe_issue_rates) run and give the
matrix-instruction costs that the MI355X's published dense peaks imply
(bf16 32x32x16: 32 cycles; the scaled 32x32x64 on FP8: 64, on FP4: 32),
which pins the cycle counting the other kinds rely on."""

import pytest

import precision_attention_forward_amd as paf

pytestmark = pytest.mark.gpu


def test_probe_mfma_costs_and_every_kind_runs(gpu):
    n = paf.load_library().attn_probe_kinds()
    costs = {}
    for kind in range(n):
        print(f"[case] probe kind {kind}", flush=True)
        paf.probe_issue_rates(kind)
        cyc, units, grid = paf.probe_issue_rates(kind)
        assert grid == 256 and units > 0 and cyc > 0
        costs[kind] = cyc / units
    for kind, expect in ((5, 32.0), (6, 64.0), (7, 32.0)):
        assert abs(costs[kind] - expect) <= 0.05 * expect, (kind, costs[kind])
    # vector instructions cost at least one cycle each; LDS kinds move at most 256 B per clock per CU
    for kind in list(range(5)) + [18, 24]:
        assert 1.0 <= costs[kind] <= 32.0, (kind, costs[kind])
    # an exponential step with work beside it costs at least the exponential alone
    for kind in range(19, 24):
        assert costs[kind] >= 0.95 * costs[1], (kind, costs[kind], costs[1])
    # MFMA with vector work beside it takes at least the MFMA time
    for kind in list(range(8, 13)) + [25, 26, 27, 28, 29]:
        assert costs[kind] >= 0.95 * 32.0, (kind, costs[kind])
    # a 128-key tile of the forward mix takes at least its 42 MFMA
    for kind in range(30, 34):
        assert costs[kind] >= 0.95 * 42 * 32.0, (kind, costs[kind])
    for kind in range(13, 18):
        assert 1.0 / costs[kind] <= 256.0 + 1.0, (kind, 1.0 / costs[kind])
