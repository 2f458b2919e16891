"""GPU parity on inputs that drive the online softmax's rarely taken paths, element by element
against the oracle.

Block-wise attention keeps a running row max and rescales what it has accumulated when a later
block raises that max ("Context Parallelism과 Expert Parallelism", §4.1, online softmax; the ring
variants merge such partials exactly, "Context Parallelism for Scalable Million-Token
Inference", §2). The bf16 MFMA kernel moves its running max only when a key tile raises it by
more than 2^8 (in base-2 units), and then rescales accumulators that already hold values. With
N(0,1) inputs and a 1/sqrt(D) scale that almost never happens after the first tile, so these
cases build inputs where it must:
  - wide score ranges: Q and K with std 3 and 6 (score std 9 and 36 nats);
  - a late spike: high-score keys in the last tiles of the KV shard a rank visits last;
  - a sink: a high-score key at the first position of a later-visited run, and at position 0;
  - early dominance: high-score first keys, later keys ramping down (the max never moves);
  - a ramp: keys score higher the later they sit, so the max climbs tile after tile.
Each runs in the partials and running (in-kernel merge) modes of ring Pass-KV at D 64 and 128,
with and without the causal mask; decode runs on the same kinds of inputs with both workspace
precisions. Bounds: bf16 inputs 2e-2 on O, 1e-3 on LSE (V stays N(0,1), so the O bound keeps
its meaning).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from ring_cases import Planted, log
from test_parity_gpu import run_decode, run_pass_kv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _chunk_edges(seqs, N, shard):
    """Global indices of the first and last token of every run the oracle puts in `shard`."""
    ranges = [(i, 0, L) for i, L in enumerate(seqs)]
    seq, pos, glob = oracle.shard_tokens(ranges, N, shard)
    starts = [0] + [i for i in range(1, len(glob))
                    if glob[i] != glob[i - 1] + 1 or seq[i] != seq[i - 1]]
    ends = [i - 1 for i in starts[1:]] + [len(glob) - 1]
    return [int(glob[i]) for i in starts], [int(glob[i]) for i in ends]


def _profile(name, seqs, N, rank, d):
    """The input generator of one named case (see the module docstring)."""
    total = int(sum(seqs))
    sd = math.sqrt(d)
    if name == "wide_std3":
        return Planted(q_std=3.0, k_std=3.0)
    if name == "wide_std6":
        return Planted(q_std=6.0, k_std=6.0)
    last = oracle.pass_kv_shard(N, rank, N - 1)          # the shard this rank visits last
    firsts, lasts = _chunk_edges(seqs, N, last)
    if name == "late_spike":
        # the last key of every run of that shard, and one a tile earlier, score ~20 nats above
        # the rest; a milder one ~6 nats above, near the threshold of the lazy max
        spikes = {g: 5.0 * sd for g in lasts}
        spikes.update({max(f, g - 64): 1.5 * sd for f, g in zip(firsts, lasts)})
        return Planted(q_bias=4.0, spikes=spikes, total=total)
    if name == "sink_later_run":
        # position 0 of the batch (visible to every query of sequence 0) and the first key of the
        # second run of the last-visited shard
        spikes = {0: 4.0 * sd}
        if len(firsts) > 1:
            spikes[firsts[1]] = 6.0 * sd
        return Planted(q_bias=4.0, spikes=spikes, total=total)
    if name == "early_dominant":
        return Planted(q_bias=4.0, spikes={0: 6.0 * sd, 1: 5.0 * sd}, ramp=-8.0 * sd, total=total)
    if name == "ramp":
        return Planted(q_bias=4.0, ramp=10.0 * sd, total=total)
    raise ValueError(name)


PROFILES = ["wide_std3", "wide_std6", "late_spike", "sink_later_run", "early_dominant", "ramp"]
SHAPES = [(128, 16, 1), (64, 8, 2)]


@pytest.mark.parametrize("mode", ["partials", "running"])
@pytest.mark.parametrize("d,n_h,n_kv", SHAPES, ids=["d128", "d64"])
@pytest.mark.parametrize("name", PROFILES)
def test_pass_kv_rescale_paths(name, d, n_h, n_kv, mode):
    seqs, N = [1500, 700], 4
    for rank in (0, N - 1):
        gen = _profile(name, seqs, N, rank, d)
        log(f"rescale case {name} d={d} mode={mode} rank={rank}")
        run_pass_kv(seqs, N, n_h, n_kv, d, "bf16", seed=21, mode=mode, ranks=[rank], std=1.0, gen=gen)


@pytest.mark.parametrize("name", ["wide_std6", "late_spike", "sink_later_run", "early_dominant"])
def test_split_running_steps_with_rescale_inputs(name):
    """Running-mode steps split over their keys (8192 tokens per rank at 2:1 heads: 64 Q tiles,
    four parts with a workspace of three partials), on inputs whose parts differ by tens of nats
    in LSE, so the in-place merge of the parts weighs one part almost alone."""
    seqs, N = [20000, 12768], 4
    for rank in (0, N - 1):
        gen = _profile(name, seqs, N, rank, 128)
        log(f"split rescale case {name} rank={rank}")
        run_pass_kv(seqs, N, 2, 1, 128, "bf16", seed=24, mode="running", ranks=[rank], std=1.0,
                    gen=gen, ws=3, n_sample=512)


@pytest.mark.parametrize("name", ["wide_std6", "late_spike", "ramp"])
def test_pass_kv_rescale_paths_without_causal_mask(name):
    seqs, N = [1100], 2
    run_pass_kv(seqs, N, 16, 1, 128, "bf16", seed=22, causal=False, mode="running", ranks=[1],
                std=1.0, gen=_profile(name, seqs, N, 1, 128))


@pytest.mark.parametrize("ws", ["f32", "bf16"])
@pytest.mark.parametrize("name", ["wide_std6", "late_spike", "ramp", "early_dominant"])
def test_decode_rescale_inputs(name, ws):
    lengths = [3000, 700, 1]
    total = sum(lengths)
    sd = math.sqrt(128)
    if name == "wide_std6":
        gen = Planted(q_std=6.0, k_std=6.0)
    elif name == "late_spike":
        # the last key of each request's cache and one 40 keys earlier
        ends = np.cumsum(lengths) - 1
        spikes = {int(e): 5.0 * sd for e in ends}
        spikes.update({int(e) - 40: 1.5 * sd for e in ends if e >= 40})
        gen = Planted(q_bias=4.0, spikes=spikes, total=total)
    elif name == "ramp":
        gen = Planted(q_bias=4.0, ramp=10.0 * sd, total=total)
    else:
        gen = Planted(q_bias=4.0, spikes={0: 6.0 * sd}, ramp=-8.0 * sd, total=total)
    run_decode(lengths, 16, 1, 128, 256, seed=23, ws=ws, gen=gen, check_splits=[0, 17, 255])
    run_decode(lengths, 16, 1, 128, 16, seed=23, ws=ws, gen=gen, check_splits=[0, 15])
