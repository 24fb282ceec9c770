"""The single-launch correction pass's bounded wait, forced from the host.

kvc_test_fused_wait withholds the matching result of one segment, so that segment's
correction items wait until the (shortened) limit, give up, and copy the segment through
with mask value 2; every kernel still runs to its end.  The rest of the launch must be
exactly what it is without the hook, and the binding must report the give-up."""
import numpy as np
import pytest
import torch

import agent_kv_cache_kvc_amd as kvc
import synth
from gpu_helpers import correct_inputs, dev, say

pytestmark = pytest.mark.gpu

WAIT_TICKS = 2_000_000  # 20 ms of the 100 MHz constant clock


@pytest.mark.parametrize("with_fb", [True, False])
def test_withheld_segment_gives_up_whole(with_fb):
    cfg = synth.CONFIGS["llama8b_t2048"].replace(L=3, H=4, T=1300, seed=91, fallback_prob=0.3)
    case = synth.generate(cfg, "cpu")
    d = dev()
    desc, _ = correct_inputs(case, d)
    ed = case.edges[0]
    K, V, U, W = (t.to(d) for t in (case.K0, case.V0, ed.U, ed.W))
    fbK = ed.exact_K.to(d) if with_fb else None
    fbV = ed.exact_V.to(d) if with_fb else None
    hold = 5
    say(f"[fused wait] {cfg.L}x{cfg.H}x{cfg.T}, withheld segment {hold}, fallback={with_fb}")
    ref = kvc.correct(K, V, desc, U, W, cfg.tau, K_fb=fbK, V_fb=fbV)
    torch.cuda.synchronize()
    kvc.lib().kvc_test_fused_wait(WAIT_TICKS, hold)
    try:
        got = kvc.correct(K, V, desc, U, W, cfg.tau, K_fb=fbK, V_fb=fbV, check=False)
        torch.cuda.synchronize()
    finally:
        kvc.lib().kvc_test_fused_wait(0, -1)
    m_ref = ref.mask.cpu().numpy().ravel()
    m = got.mask.cpu().numpy().ravel()
    assert m[hold] == 2
    others = np.arange(m.size) != hold
    np.testing.assert_array_equal(m[others], m_ref[others])
    l, h = divmod(hold, cfg.H)
    for name, out, src, fb, r in (("K", got.K, K, fbK, ref.K), ("V", got.V, V, fbV, ref.V)):
        want = (fb if fb is not None else src)[l, h]
        assert torch.equal(out[l, h], want), f"{name}: withheld segment is not the copy-through"
        sel = torch.ones(cfg.L, cfg.H, dtype=torch.bool)
        sel[l, h] = False
        assert torch.equal(out[sel.to(d)], r[sel.to(d)]), f"{name}: other segments changed"
    with pytest.raises(kvc.KvcWaitError):
        kvc.check_mask(got.mask)
    # the hook is off again: the same launch gives the reference result
    again = kvc.correct(K, V, desc, U, W, cfg.tau, K_fb=fbK, V_fb=fbV)
    torch.cuda.synchronize()
    assert torch.equal(again.mask, ref.mask) and torch.equal(again.K, ref.K)
