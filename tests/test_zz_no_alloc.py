"""The allocation-free decode entry point (cp_decode_splitkv_noalloc) against the workspace entry
point it varies (cp_decode_splitkv / cp_decode_splitkv_ex), through the C ABI on the GPU.

Two calls in a row, the second with a smaller input, for each workspace precision: the library's
scratch array keeps the first call's partials, so the second call must not depend on them. Both
entry points run the same kernels, which are deterministic, so their outputs must agree bit for
bit (a stronger bar than the oracle's bounds, which the decode parity tests check)."""
import numpy as np
import pytest
import torch

import synth_inputs as si
from ring_cases import device_tensor, log, scale_of

pytestmark = pytest.mark.gpu


def _decode_pair(lengths, n_h, n_kv, d, S, ws, seed):
    from context_ring_attention_amd import binding as cp
    lengths = np.asarray(lengths, np.int64)
    B = len(lengths)
    offs = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    toks = np.arange(int(lengths.sum()))
    kc = device_tensor(seed, si.TID_K, toks, (n_kv, d), 1.0, "bf16")
    vc = device_tensor(seed, si.TID_V, toks, (n_kv, d), 1.0, "bf16")
    q = device_tensor(seed, si.TID_Q, np.arange(B), (n_h, d), 1.0, "bf16")
    offs_d, lens_d = torch.from_numpy(offs).cuda(), torch.from_numpy(lengths).cuda()
    scale = scale_of(d)
    ws_o, ws_l = cp.decode_workspace(B, n_h, d, S, ws_dtype=ws)
    o_ref = torch.full((B, n_h, d), float("nan"), device="cuda")
    l_ref = torch.full((B, n_h), float("nan"), device="cuda")
    cp.decode_splitkv(q, kc, vc, offs_d, lens_d, S, scale, ws_o, ws_l, o_ref, l_ref)
    o = torch.full((B, n_h, d), float("nan"), device="cuda")
    lse = torch.full((B, n_h), float("nan"), device="cuda")
    cp.decode_splitkv_noalloc(q, kc, vc, offs_d, lens_d, S, scale, o, lse, ws_dtype=ws)
    torch.cuda.synchronize()
    log(f"noalloc decode B={B} S={S} n_h={n_h} d={d} ws={ws}: "
        f"max|dO|={float((o - o_ref).abs().max()):.3e}")
    assert torch.equal(o, o_ref), "O differs from the workspace entry point"
    assert torch.equal(lse, l_ref), "LSE differs from the workspace entry point"
    assert bool(torch.isfinite(o).all())


@pytest.mark.parametrize("ws", ["f32", "bf16"])
def test_noalloc_decode_matches_workspace_entry_point_on_two_calls(ws):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # first call: 32 requests x 256 splits x 16 heads x D 128 (the largest workspace the array is
    # sized for, at fp32), then a smaller one with fewer splits, GQA and D 64
    lens = [int(x) for x in np.random.default_rng(40).integers(1, 2500, size=32)]
    lens[3] = 0
    _decode_pair(lens, 16, 1, 128, 256, ws, seed=41)
    _decode_pair([700, 1, 129], 8, 2, 64, 16, ws, seed=42)
