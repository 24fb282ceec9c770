"""The Python binding checks every caller-supplied tensor (shape, dtype, device, contiguity)
before it hands a pointer to the library: a wrong output or workspace raises here, on the
host, and no kernel is ever launched with it.  CPU tensors stand in for device memory; every
case below fails before the first call into the library's compute entry points."""
import pytest
import torch

import agent_kv_cache_kvc_amd as kvc

L, H, T, d, A, r = 2, 2, 8, 64, 2, 4


def _case(dtype=torch.bfloat16):
    z = dict(dtype=dtype)
    K = torch.zeros(L, H, T, d, **z)
    V = torch.zeros(L, H, T, d, **z)
    ed = dict(desc=torch.zeros(L, H, A, 2 * d), U=torch.zeros(2, L, H, A, T, r, **z),
              W=torch.zeros(2, L, H, A, r, d, **z))
    return K, V, ed


def _bad_outputs():
    K, _, _ = _case()
    return [
        ("shape", torch.zeros(L, H, T + 1, d, dtype=K.dtype), ValueError),
        ("dtype", torch.zeros(L, H, T, d, dtype=torch.float32), TypeError),
        ("contiguous", torch.zeros(L, H, d, T, dtype=K.dtype).transpose(-1, -2), ValueError),
        ("device", torch.zeros(L, H, T, d, dtype=K.dtype, device="meta"), ValueError),
    ]


@pytest.mark.parametrize("which", range(4))
def test_chain_checks_caller_outputs(which):
    K, V, ed = _case()
    name, bad, exc = _bad_outputs()[which]
    good = torch.zeros_like(K)
    with pytest.raises(exc):
        kvc.correct_chain(K, V, [ed, ed], 0.3, outputs=[(good, good.clone()), (good.clone(), bad)])


def test_chain_checks_source_and_output_count():
    K, V, ed = _case()
    with pytest.raises(ValueError, match="contiguous"):
        kvc.correct_chain(K.transpose(0, 1).contiguous().transpose(0, 1), V, [ed], 0.3)
    with pytest.raises(ValueError, match="pairs"):
        kvc.correct_chain(K, V, [ed, ed], 0.3, outputs=[(K.clone(), V.clone())])


@pytest.mark.parametrize("which", range(4))
def test_fanout_checks_caller_outputs(which):
    K, V, ed = _case()
    name, bad, exc = _bad_outputs()[which]
    with pytest.raises(exc):
        kvc.correct_fanout(K, V, [ed, ed], 0.3,
                           outputs=[(bad, torch.zeros_like(K)), (torch.zeros_like(K), torch.zeros_like(K))])


@pytest.mark.parametrize("which", range(4))
def test_pooled_checks_caller_outputs(which):
    K, V, _ = _case()
    pool = kvc.AnchorPool.empty(L, H, T, d, 3, r, dtype=K.dtype, device="cpu")
    name, bad, exc = _bad_outputs()[which]
    with pytest.raises(exc):
        kvc.correct_pooled(K, V, pool, A, 0.3, K_out=torch.zeros_like(K), V_out=bad)


@pytest.mark.parametrize("which", range(4))
def test_correct_checks_caller_outputs(which):
    K, V, ed = _case()
    name, bad, exc = _bad_outputs()[which]
    with pytest.raises(exc):
        kvc.correct(K, V, ed["desc"], ed["U"], ed["W"], 0.3, K_out=bad)


def test_workspace_device_and_layout_are_checked():
    K, V, ed = _case()
    ws_meta = torch.empty(1 << 20, dtype=torch.uint8, device="meta")
    with pytest.raises(ValueError, match="workspace must be on"):
        kvc.correct(K, V, ed["desc"], ed["U"], ed["W"], 0.3, workspace=ws_meta)
    with pytest.raises(ValueError, match="workspace must be on"):
        kvc.correct_chain(K, V, [ed], 0.3, workspace=ws_meta)
    with pytest.raises(ValueError, match="workspace must be on"):
        kvc.fit_anchor(torch.zeros(4, T, d, dtype=K.dtype), r=4, workspace=ws_meta)
    strided = torch.empty(1 << 21, dtype=torch.uint8)[::2]
    with pytest.raises(ValueError, match="workspace must be contiguous"):
        kvc.correct_fanout(K, V, [ed, ed], 0.3, workspace=strided)


def test_workspace_size_is_passed_in_bytes():
    ws = torch.empty(64, dtype=torch.float32)
    assert kvc._ws_bytes(ws) == 256
