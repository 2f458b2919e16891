"""Repeatability and stream independence of the HIP path, through the C ABI (GPU).

- Every kernel reduces in a fixed order (tile order, split order, fixed LDS reduction trees), so
  the same call on the same inputs must give bitwise the same outputs, whatever garbage the
  output buffers held before. Checked for ring Pass-KV (kept partials and running merge, which
  reads its previous output), ring Pass-Q, the LSE merge and split-KV decode.
- The library keeps no device state between calls: a ring and a decode enqueued at once on two
  streams of default priority must each give bitwise the result it gives alone.
"""
import numpy as np
import pytest
import torch

import synth_inputs as si
from ring_cases import device_tensor, log, product_shards, scale_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from context_ring_attention_amd import binding
    binding.load()


def _bits(t):
    return t.contiguous().view(torch.int32) if t.dtype == torch.float32 else t.contiguous().view(torch.int16)


def _same(a, b, what):
    assert a.shape == b.shape and torch.equal(_bits(a), _bits(b)), f"{what}: not bitwise identical"


class Ring:
    """A bf16 Pass-KV ring of one rank: 3000 + 1001 tokens, CP 4, 16:1 heads, D = 128."""

    def __init__(self, seed=0, N=4, rank=1, n_h=16, n_kv=1, d=128):
        ranges = [(0, 0, 3000), (1, 0, 1001)]
        self.N, self.rank, self.n_h, self.d = N, rank, n_h, d
        self.sh = product_shards(ranges, N)
        for s in self.sh.values():
            s.k = device_tensor(seed, si.TID_K, s.tokens, (n_kv, d), 1.0, "bf16")
            s.v = device_tensor(seed, si.TID_V, s.tokens, (n_kv, d), 1.0, "bf16")
            s.q = device_tensor(seed, si.TID_Q, s.tokens, (n_h, d), 1.0, "bf16")
        self.tq = self.sh[rank].q.shape[0]

    def run(self, mode, stream=None):
        from context_ring_attention_amd import binding as cp
        N, r, tq = self.N, self.rank, self.tq
        o = torch.full((tq, self.n_h, self.d), float("nan"), device="cuda")
        lse = torch.full((tq, self.n_h), 7.0, device="cuda")
        kw = {}
        if mode == "partials":
            kw["o_parts"] = [torch.full_like(o, 3.0) for _ in range(N)]
            kw["lse_parts"] = [torch.full_like(lse, -1.0) for _ in range(N)]
        else:
            kw["o_acc"], kw["lse_acc"] = o, lse
        sh = self.sh
        cp.ring_pass_kv(sh[r].q, sh[r].segs, r, [sh[s].k for s in range(N)], [sh[s].v for s in range(N)],
                        [sh[s].segs for s in range(N)], True, scale_of(self.d), o, lse, stream=stream, **kw)
        return o, lse

    def run_pass_q(self):
        from context_ring_attention_amd import binding as cp
        N, sh = self.N, self.sh
        parts_o = [torch.full((sh[i // N].q.shape[0], self.n_h, self.d), 5.0, device="cuda") for i in range(N * N)]
        parts_l = [torch.full((sh[i // N].q.shape[0], self.n_h), 2.0, device="cuda") for i in range(N * N)]
        outs = [torch.full((sh[i].q.shape[0], self.n_h, self.d), float("nan"), device="cuda") for i in range(N)]
        lses = [torch.empty(sh[i].q.shape[0], self.n_h, device="cuda") for i in range(N)]
        cp.ring_pass_q([sh[i].q for i in range(N)], [sh[i].segs for i in range(N)],
                       [sh[i].k for i in range(N)], [sh[i].v for i in range(N)],
                       [sh[i].segs for i in range(N)], True, scale_of(self.d), parts_o, parts_l, outs, lses)
        return outs + lses


class Decode:
    """Split-KV decode of 40 requests (enough units for one wave per split), 256 splits."""

    def __init__(self, seed=1, n_h=16, n_kv=1, d=128, S=256):
        lengths = np.random.default_rng(11).integers(1, 6000, size=40).astype(np.int64)
        self.B, self.S, self.n_h, self.d = len(lengths), S, n_h, d
        offs = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
        toks = np.arange(int(lengths.sum()))
        self.kc = device_tensor(seed, si.TID_K, toks, (n_kv, d), 1.0, "bf16")
        self.vc = device_tensor(seed, si.TID_V, toks, (n_kv, d), 1.0, "bf16")
        self.q = device_tensor(seed, si.TID_Q, np.arange(self.B), (n_h, d), 1.0, "bf16")
        self.offs = torch.from_numpy(offs).cuda()
        self.lens = torch.from_numpy(lengths).cuda()

    def run(self, stream=None):
        from context_ring_attention_amd import binding as cp
        ws_o, ws_l = cp.decode_workspace(self.B, self.n_h, self.d, self.S)
        ws_o.fill_(1.5)
        ws_l.fill_(-2.0)
        o = torch.full((self.B, self.n_h, self.d), float("nan"), device="cuda")
        lse = torch.empty(self.B, self.n_h, device="cuda")
        cp.decode_splitkv(self.q, self.kc, self.vc, self.offs, self.lens, self.S, scale_of(self.d),
                          ws_o, ws_l, o, lse, stream=stream)
        return o, lse, ws_o, ws_l


def test_ring_merge_and_decode_are_bitwise_repeatable():
    ring, dec = Ring(), Decode()
    for mode in ("partials", "running"):
        log(f"ring pass-kv {mode}, twice")
        a = ring.run(mode)
        b = ring.run(mode)
        torch.cuda.synchronize()
        for x, y, name in zip(a, b, ("O", "LSE")):
            _same(x, y, f"pass-kv {mode} {name}")
    log("ring pass-q (16 partials + 4 merges), twice")
    for i, (x, y) in enumerate(zip(ring.run_pass_q(), ring.run_pass_q())):
        _same(x, y, f"pass-q output {i}")
    log("decode B=40 S=256, twice")
    a, b = dec.run(), dec.run()
    torch.cuda.synchronize()
    for x, y, name in zip(a, b, ("O", "LSE", "split O", "split LSE")):
        _same(x, y, f"decode {name}")


def test_split_ring_steps_are_bitwise_repeatable():
    """Running-mode Pass-KV steps split over their keys (four parts through a ring workspace of
    three partials): two calls whose workspaces start with different garbage give the same bits
    (the partials start from a filled empty result, the merge order is fixed)."""
    from context_ring_attention_amd import binding as cp
    N, r, n_h, n_kv, d = 4, 1, 1, 1, 128
    sh = product_shards([(0, 0, 32768)], N)
    for s in sh.values():
        s.k = device_tensor(7, si.TID_K, s.tokens, (n_kv, d), 1.0, "bf16")
        s.v = device_tensor(7, si.TID_V, s.tokens, (n_kv, d), 1.0, "bf16")
    q = device_tensor(7, si.TID_Q, sh[r].tokens, (n_h, d), 1.0, "bf16")
    outs = []
    for fill in (0, 255):
        ws = cp.ring_workspace(q.shape[0], n_h, d, partials=3)
        ws.fill_(fill)
        o = torch.full((q.shape[0], n_h, d), float("nan"), device="cuda")
        lse = torch.full((q.shape[0], n_h), 7.0, device="cuda")
        log(f"split running pass-kv, workspace filled with {fill}")
        cp.ring_pass_kv(q, sh[r].segs, r, [sh[s].k for s in range(N)], [sh[s].v for s in range(N)],
                        [sh[s].segs for s in range(N)], True, scale_of(d), o, lse, o_acc=o, lse_acc=lse,
                        workspace=ws)
        outs.append((o, lse))
    torch.cuda.synchronize()
    for x, y, name in zip(outs[0], outs[1], ("O", "LSE")):
        _same(x, y, f"split pass-kv {name}")
    assert torch.isfinite(outs[0][0]).all()


def test_concurrent_streams_match_serial_results():
    ring, dec = Ring(seed=2, rank=3), Decode(seed=3)
    ref_ring = ring.run("running")
    ref_dec = dec.run()
    torch.cuda.synchronize()
    main = torch.cuda.current_stream()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    s1.wait_stream(main)
    s2.wait_stream(main)
    log("ring on one stream, decode on another, enqueued together")
    with torch.cuda.stream(s1):
        got_ring = ring.run("running", stream=s1)
    with torch.cuda.stream(s2):
        got_dec = dec.run(stream=s2)
    torch.cuda.synchronize()
    for x, y, name in zip(ref_ring, got_ring, ("O", "LSE")):
        _same(x, y, f"ring {name} (concurrent)")
    for x, y, name in zip(ref_dec, got_dec, ("O", "LSE", "split O", "split LSE")):
        _same(x, y, f"decode {name} (concurrent)")
