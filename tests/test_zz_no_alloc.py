"""kvc_correct_noalloc (the correction with the library's own device scratch array instead of a
caller workspace) against kvc_correct on the same inputs, through the C ABI: two calls in a
row, the second on a smaller cache, both bit for bit; a shape whose workspace exceeds the
scratch array is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import agent_kv_cache_kvc_amd as kvc
import synth
from gpu_helpers import correct_inputs, dev, say

pytestmark = pytest.mark.gpu


def _noalloc(K, V, desc, U, W, tau, K_fb=None, V_fb=None):
    L, H, T, d = K.shape
    A, r = desc.shape[2], U.shape[-1]
    Ko, Vo = torch.empty_like(K), torch.empty_like(V)
    mask = torch.empty(L, H, dtype=torch.uint8, device=K.device)
    score = torch.empty(L, H, dtype=torch.float32, device=K.device)
    w = torch.empty(L, H, A, dtype=torch.float32, device=K.device)
    qn = torch.empty(L, H, 2 * d, dtype=torch.float32, device=K.device)
    p = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    st = kvc.lib().kvc_correct_noalloc(
        p(K), p(V), L, H, T, d, kvc._dtype_code(K), p(desc), p(U), p(W), A, r,
        ctypes.c_float(tau), None, p(K_fb), p(V_fb), p(Ko), p(Vo), p(mask), p(score), p(w),
        p(qn), torch.cuda.current_stream(K.device).cuda_stream)
    assert st == 0, kvc.lib().kvc_last_error().decode()
    return Ko, Vo, mask, score, w, qn


@pytest.mark.parametrize("shapes", [((8, 8, 1500, 4, 32, "bf16"), (2, 3, 300, 2, 16, "bf16")),
                                    ((4, 4, 700, 2, 128, "bf16"), (1, 2, 129, 3, 8, "f32"))])
def test_noalloc_matches_kvc_correct_on_two_calls(shapes):
    d = dev()
    for i, (L, H, T, A, r, dt) in enumerate(shapes):
        cfg = synth.CONFIGS["llama8b_t2048"].replace(name=f"noalloc{i}", L=L, H=H, T=T, A=A,
                                                     r=r, dtype=dt, seed=700 + i,
                                                     fallback_prob=0.3)
        say(f"[noalloc] call {i}: {L}x{H}x{T} A={A} r={r} {dt}")
        case = synth.generate(cfg, "cpu")
        desc, _ = correct_inputs(case, d)
        ed = case.edges[0]
        K, V, U, W = (t.to(d) for t in (case.K0, case.V0, ed.U, ed.W))
        fbK, fbV = ed.exact_K.to(d), ed.exact_V.to(d)
        ref = kvc.correct(K, V, desc, U, W, cfg.tau, K_fb=fbK, V_fb=fbV, want_q_next=True)
        got = _noalloc(K, V, desc, U, W, cfg.tau, fbK, fbV)
        torch.cuda.synchronize()
        Ko, Vo, mask, score, w, qn = got
        assert torch.equal(mask, ref.mask) and int(mask.max()) <= 1
        assert torch.equal(Ko, ref.K) and torch.equal(Vo, ref.V)
        assert torch.equal(score, ref.score) and torch.equal(w, ref.w)
        assert torch.equal(qn, ref.q_next)
        say(f"  bit for bit: mask {mask.cpu().numpy().ravel().tolist()[:12]}")


def test_noalloc_refuses_a_workspace_above_the_scratch_array():
    lib = kvc.lib()
    FAKE = 0x10000
    L, H, T, d, A, r = 32, 8, 8192, 128, 4, 32
    need = lib.kvc_correct_workspace_bytes(L, H, T, d, A, r)
    assert need > 16 << 20
    st = lib.kvc_correct_noalloc(FAKE, FAKE, L, H, T, d, 0, FAKE, FAKE, FAKE, A, r,
                                 ctypes.c_float(0.3), None, None, None, FAKE, FAKE, FAKE, None,
                                 None, None, None)
    assert st == 2 and "scratch" in lib.kvc_last_error().decode()
