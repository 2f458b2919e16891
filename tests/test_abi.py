"""C-ABI checks that need no GPU: the library loads, exports every declared entry point, the
host-only shard map matches the oracle bit for bit, and invalid arguments are rejected with the
documented status before anything is launched."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from context_ring_attention_amd import binding as cp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cpattn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cp_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = cp.load()
    names = _declared_functions()
    assert set(names) >= {"cp_shard_map", "cp_partial_attn", "cp_merge_lse", "cp_decode_splitkv"}
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(cp.EXPORTED)


def _oracle_segments(ranges, N, r):
    seq, pos, glob = oracle.shard_tokens(ranges, N, r)
    return seq, pos, glob


def _expand(segs):
    seq, pos, loc = [], [], []
    for s, p, n, l in segs:
        seq += [s] * n
        pos += list(range(p, p + n))
        loc += list(range(l, l + n))
    return np.array(seq, np.int64), np.array(pos, np.int64), np.array(loc, np.int64)


CASES = [
    ([(0, 0, 256)], 4),                                         # the tiny ring
    ([(0, 0, 128 * 1024)], 4),                                  # 128K at CP4
    ([(0, 0, 120 * 1024), (0, 120 * 1024, 128 * 1024)], 4),     # cached prefix + new tokens
    ([(0, 120 * 1024, 128 * 1024)], 4),                         # the new tokens alone
    ([(i, 0, L) for i, L in enumerate([64 * 1024, 192 * 1024, 256 * 1024, 512 * 1024])], 8),
    ([(0, 0, 257), (1, 0, 3), (2, 0, 0), (3, 5, 13)], 4),        # ragged and degenerate ranges
    ([(2, 0, 10), (0, 0, 7)], 3),                               # ids out of order, a missing id
    ([(0, 0, 1)], 1),
]


@pytest.mark.parametrize("ranges,N", CASES)
def test_shard_map_bit_exact_against_oracle(ranges, N):
    for r in range(N):
        segs, toks = cp.shard_map(ranges, N, r)
        seq, pos, loc = _expand(segs)
        oseq, opos, oglob = _oracle_segments(ranges, N, r)
        assert np.array_equal(seq, oseq) and np.array_equal(pos, opos)
        assert np.array_equal(loc, np.arange(len(loc)))
        assert np.array_equal(toks, oglob)
        assert all(n > 0 for _, _, n, _ in segs)   # empty chunks are not emitted


def test_shard_map_capacity_and_argument_errors():
    lib = cp.load()
    i64p = ctypes.POINTER(ctypes.c_int64)
    b = np.array([0], np.int64)
    e = np.array([256], np.int64)
    n_segs = ctypes.c_int(0)
    n_tok = ctypes.c_int64(0)
    segs = (cp.CpSegment * 1)()
    st = lib.cp_shard_map(1, None, b.ctypes.data_as(i64p), e.ctypes.data_as(i64p), 4, 1, segs, 1,
                          ctypes.byref(n_segs), None, 0, ctypes.byref(n_tok))
    assert st == cp.CP_E_CAPACITY and n_segs.value == 2 and n_tok.value == 64
    st = lib.cp_shard_map(1, None, b.ctypes.data_as(i64p), e.ctypes.data_as(i64p), 4, 4, segs, 1,
                          ctypes.byref(n_segs), None, 0, None)
    assert st == cp.CP_E_ARG and "rank" in cp.last_error()
    bad_e = np.array([-1], np.int64)
    st = lib.cp_shard_map(1, None, b.ctypes.data_as(i64p), bad_e.ctypes.data_as(i64p), 4, 0, segs, 1,
                          ctypes.byref(n_segs), None, 0, None)
    assert st == cp.CP_E_ARG
    # a range whose chunk edges c * L / 2N would overflow 64 bits
    huge_e = np.array([1 << 62], np.int64)
    st = lib.cp_shard_map(1, None, b.ctypes.data_as(i64p), huge_e.ctypes.data_as(i64p), 4, 0, segs, 1,
                          ctypes.byref(n_segs), None, 0, None)
    assert st == cp.CP_E_UNSUPPORTED and "too large" in cp.last_error()


def _partial(**kw):
    lib = cp.load()
    seg, n = cp.segments([(0, 0, 16, 0)])
    args = dict(q=16, k=16, v=16, tq=16, tk=16, n_h=4, n_kv=1, d_h=64, dt=cp.CP_BF16, qs=seg, nq=n,
                ks=seg, nk=n, causal=1, scale=0.125, o=16, lse=16, acc=0)
    args.update(kw)
    return lib.cp_partial_attn(args["q"], args["k"], args["v"], args["tq"], args["tk"], args["n_h"],
                               args["n_kv"], args["d_h"], args["dt"], args["qs"], args["nq"],
                               args["ks"], args["nk"], args["causal"], args["scale"], args["o"],
                               args["lse"], args["acc"], None)


def test_partial_attn_rejects_bad_arguments_without_launching():
    assert _partial(n_h=6, n_kv=4) == cp.CP_E_SHAPE
    assert _partial(d_h=96) == cp.CP_E_UNSUPPORTED
    assert _partial(dt=7) == cp.CP_E_ARG
    assert _partial(scale=0.0) == cp.CP_E_ARG
    assert _partial(scale=float("nan")) == cp.CP_E_ARG
    assert _partial(acc=2) == cp.CP_E_ARG
    assert _partial(q=0) == cp.CP_E_ARG
    assert _partial(q=8) == cp.CP_E_ARG            # not 16-byte aligned
    big, n = cp.segments([(0, 0, 17, 0)])
    assert _partial(qs=big, nq=n) == cp.CP_E_SHAPE   # runs past the shard
    assert "outside the shard" in cp.last_error()
    # tables longer than one launch takes are accepted (split over launches); nothing to do with
    # no query run, so nothing is launched here
    many, n = cp.segments([(0, i, 1, 0) for i in range(65)])
    assert _partial(ks=many, nk=n, nq=0) == cp.CP_OK
    bad_many, n = cp.segments([(0, i, 1, 0) for i in range(64)] + [(0, 0, 17, 0)])
    assert _partial(ks=bad_many, nk=n) == cp.CP_E_SHAPE         # every run is still validated
    neg, n = cp.segments([(-1, 0, 1, 0)])
    assert _partial(ks=neg, nk=n) == cp.CP_E_SHAPE
    assert _partial(tq=1 << 31) == cp.CP_E_UNSUPPORTED
    huge, n = cp.segments([(0, 0, 1 << 27, 0)])       # 2^27 tokens x 16 heads per KV head
    assert _partial(qs=huge, nq=n, tq=1 << 27, n_h=16, n_kv=1) == cp.CP_E_UNSUPPORTED
    # fields whose sums would overflow 64 bits are rejected, not wrapped
    wrap, n = cp.segments([(0, 0, 1 << 62, 1 << 62)])
    assert _partial(qs=wrap, nq=n) == cp.CP_E_SHAPE
    far, n = cp.segments([(0, (1 << 63) - 1, 1, 0)])
    assert _partial(ks=far, nk=n) == cp.CP_E_UNSUPPORTED
    # nothing to do is not an error (no launch either)
    assert _partial(nq=0) == cp.CP_OK


def _partial_bwd(**kw):
    lib = cp.load()
    seg, n = cp.segments([(0, 0, 16, 0)])
    args = dict(q=16, k=16, v=16, tq=16, tk=16, n_h=4, n_kv=1, d_h=64, dt=cp.CP_BF16, qs=seg, nq=n,
                ks=seg, nk=n, causal=1, scale=0.125, lse=16, delta=16, d_o=16, dq=16, dk=16, dv=16,
                ws=None, ws_bytes=0)
    args.update(kw)
    return lib.cp_partial_attn_bwd(args["q"], args["k"], args["v"], args["tq"], args["tk"],
                                   args["n_h"], args["n_kv"], args["d_h"], args["dt"], args["qs"],
                                   args["nq"], args["ks"], args["nk"], args["causal"], args["scale"],
                                   args["lse"], args["delta"], args["d_o"], args["dq"], args["dk"],
                                   args["dv"], args["ws"], args["ws_bytes"], None)


def test_backward_workspace_size_and_argument_checks():
    """The backward workspace bound is fixed per head dimension (2048 slots of 128 keys x d_h x
    dK and dV in fp32); bad backward arguments fail before any launch (fake pointers here)."""
    assert cp.attn_bwd_workspace_bytes(128) == 2048 * 128 * 128 * 4 * 2
    assert cp.attn_bwd_workspace_bytes(64) == 2048 * 128 * 64 * 4 * 2
    assert cp.attn_bwd_workspace_bytes(96) == 0
    assert _partial_bwd(ws=0x7000008, ws_bytes=1 << 20) == cp.CP_E_ARG   # misaligned workspace
    assert "workspace" in cp.last_error()
    assert _partial_bwd(dt=7) == cp.CP_E_ARG
    assert _partial_bwd(dk=0) == cp.CP_E_ARG
    assert _partial_bwd(d_o=8) == cp.CP_E_ARG                            # not 16-byte aligned
    assert _partial_bwd(n_h=6, n_kv=4) == cp.CP_E_SHAPE
    assert _partial_bwd(nq=0) == cp.CP_OK                                 # nothing to do
    # the ring driver checks the workspace before its first launch (the delta kernel)
    lib = cp.load()
    N = 2
    a = _ring_arrays(N)
    vp = ctypes.c_void_p
    dks = (vp * N)(*[0x7300000 + 0x100000 * i for i in range(N)])
    st = lib.cp_ring_pass_kv_bwd(a["q"][0], 16, a["q_segs"][0], 1, N, 0, a["k"], a["v"], a["tk"],
                                 a["kv_segs"], a["nk"], 16, 1, 128, cp.CP_BF16, 1, 0.1, 0x7000000,
                                 0x7100000, 0x7200000, 0x7400000, 0x7500000, dks, dks, 0x7600008,
                                 1 << 20, None)
    assert st == cp.CP_E_ARG and "workspace" in cp.last_error()


def test_merge_and_decode_reject_bad_arguments():
    lib = cp.load()
    vp = ctypes.c_void_p
    parts = (vp * 1)(16)
    assert lib.cp_merge_lse(0, parts, parts, 8, 64, 16, cp.CP_F32, None, None) == cp.CP_E_CAPACITY
    assert lib.cp_merge_lse(65, parts, parts, 8, 64, 16, cp.CP_F32, None, None) == cp.CP_E_CAPACITY
    assert lib.cp_merge_lse(1, parts, parts, 8, 80, 16, cp.CP_F32, None, None) == cp.CP_E_UNSUPPORTED
    assert lib.cp_merge_lse(1, parts, parts, 8, 64, 16, cp.CP_BF16, None, None) == cp.CP_E_ARG  # alias
    assert lib.cp_merge_lse(1, parts, parts, 0, 64, 32, cp.CP_F32, None, None) == cp.CP_OK
    dec = lib.cp_decode_splitkv
    assert dec(16, 16, 16, 16, 16, 2, 16, 1, 128, cp.CP_F32, 256, 0.1, 16, 16, 16, cp.CP_F32, None,
               None) == cp.CP_E_UNSUPPORTED
    assert dec(16, 16, 16, 16, 16, 2, 16, 1, 128, cp.CP_BF16, 0, 0.1, 16, 16, 16, cp.CP_F32, None,
               None) == cp.CP_E_UNSUPPORTED
    assert dec(16, 16, 16, 16, 16, 2, 16, 3, 128, cp.CP_BF16, 256, 0.1, 16, 16, 16, cp.CP_F32, None,
               None) == cp.CP_E_SHAPE
    assert dec(0, 16, 16, 16, 16, 2, 16, 1, 128, cp.CP_BF16, 256, 0.1, 16, 16, 16, cp.CP_F32, None,
               None) == cp.CP_E_ARG
    # fp32 partial O, then fp32 LSE; the _ex sizes follow the chosen workspace dtype
    assert lib.cp_decode_workspace_bytes(32, 16, 128, 256) == 32 * 256 * 16 * (128 * 4 + 4)
    assert lib.cp_decode_workspace_bytes_ex(32, 16, 128, 256, cp.CP_F32) == 32 * 256 * 16 * (128 * 4 + 4)
    assert lib.cp_decode_workspace_bytes_ex(32, 16, 128, 256, cp.CP_BF16) == 32 * 256 * 16 * (128 * 2 + 4)
    assert lib.cp_decode_workspace_bytes_ex(32, 16, 128, 256, 7) == 0
    dex = lib.cp_decode_splitkv_ex
    assert dex(16, 16, 16, 16, 16, 2, 16, 1, 128, cp.CP_BF16, 256, 0.1, 7, 16, 16, 16, cp.CP_F32, None,
               None) == cp.CP_E_ARG                                    # bad workspace dtype
    assert dex(16, 16, 16, 16, 16, 2, 16, 1, 128, cp.CP_BF16, 2000, 0.1, cp.CP_BF16, 16, 16, 16,
               cp.CP_F32, None, None) == cp.CP_E_UNSUPPORTED
    # the allocation-free variant rejects a workspace beyond its array before any device call
    noalloc = lib.cp_decode_splitkv_noalloc
    assert noalloc(16, 16, 16, 16, 16, 64, 16, 1, 128, cp.CP_BF16, 256, 0.1, cp.CP_F32, 16, cp.CP_F32,
                   None, None) == cp.CP_E_CAPACITY
    assert "scratch array" in cp.last_error()
    assert noalloc(16, 16, 16, 16, 16, 0, 16, 1, 128, cp.CP_BF16, 256, 0.1, cp.CP_F32, 16, cp.CP_F32,
                   None, None) == cp.CP_OK                             # nothing to do, no lookup
    assert noalloc(16, 16, 16, 16, 16, 2, 16, 1, 128, cp.CP_BF16, 256, 0.1, 9, 16, cp.CP_F32,
                   None, None) == cp.CP_E_ARG
    assert lib.cp_decode_workspace_bytes(32, 16, 128, 256) <= cp.CP_DECODE_NOALLOC_MAX_BYTES
    # grid limits are checked on the host: one merge workgroup of 256 threads per (request, head)
    assert dec(16, 16, 16, 16, 16, 65535, 4096, 4096, 128, cp.CP_BF16, 256, 0.1, 16, 16, 16,
               cp.CP_F32, None, None) == cp.CP_E_UNSUPPORTED
    assert lib.cp_status_string(cp.CP_E_HIP) == b"CP_E_HIP"


def _ring_arrays(N, tq=16, tk=16, bad_kv=None, bad_o_out=False):
    """ctypes arrays for the ring drivers with fake (never dereferenced) 16-byte aligned device
    pointers; shard `bad_kv` gets a run that overflows its shard."""
    vp = ctypes.c_void_p
    segp = ctypes.POINTER(cp.CpSegment)
    good, _ = cp.segments([(0, 0, tq, 0)])
    kv_ok, _ = cp.segments([(0, 0, tk, 0)])
    kv_bad, _ = cp.segments([(0, 0, tk + 1, 0)])
    ptr = lambda i: 0x100000 + 0x1000 * i
    a = {
        "q": (vp * N)(*[ptr(i) for i in range(N)]),
        "tq": (ctypes.c_int64 * N)(*[tq] * N),
        "q_segs": (segp * N)(*[ctypes.cast(good, segp)] * N),
        "nq": (ctypes.c_int * N)(*[1] * N),
        "k": (vp * N)(*[ptr(100 + i) for i in range(N)]),
        "v": (vp * N)(*[ptr(200 + i) for i in range(N)]),
        "tk": (ctypes.c_int64 * N)(*[tk] * N),
        "kv_segs": (segp * N)(*[ctypes.cast(kv_bad if i == bad_kv else kv_ok, segp) for i in range(N)]),
        "nk": (ctypes.c_int * N)(*[1] * N),
        "o_parts": (vp * (N * N))(*[ptr(300 + i) for i in range(N * N)]),
        "l_parts": (vp * (N * N))(*[ptr(400 + i) for i in range(N * N)]),
        "o_out": (vp * N)(*[None if (bad_o_out and i == N - 1) else ptr(500 + i) for i in range(N)]),
    }
    return a


def test_ring_drivers_validate_every_step_and_merge_before_launching():
    """A bad shard reached only at a late ring step, or a bad final-merge output, must fail the
    call before anything is launched (the pointers here are fake; a launch would fault)."""
    lib = cp.load()
    N = 4
    # Pass-KV, rank 0: shard 3 is visited at step 1, shard 1 at the last step
    for bad in (1, 3):
        a = _ring_arrays(N, bad_kv=bad)
        st = lib.cp_ring_pass_kv(a["q"][0], 16, a["q_segs"][0], 1, N, 0, a["k"], a["v"], a["tk"], a["kv_segs"],
                                 a["nk"], 16, 1, 128, cp.CP_BF16, 1, 0.1, None, None, 0x7000000,
                                 0x7100000, 0x7200000, cp.CP_BF16, None, None, 0, None)
        assert st == cp.CP_E_SHAPE and "kv_segs" in cp.last_error()
    # Pass-KV partials mode with a NULL part: caught by the merge check, before any launch
    a = _ring_arrays(N)
    parts = a["o_parts"]
    parts[2] = None
    st = lib.cp_ring_pass_kv(a["q"][0], 16, a["q_segs"][0], 1, N, 0, a["k"], a["v"], a["tk"], a["kv_segs"],
                             a["nk"], 16, 1, 128, cp.CP_BF16, 1, 0.1, parts, a["l_parts"], None, None,
                             0x7200000, cp.CP_F32, None, None, 0, None)
    assert st == cp.CP_E_ARG
    # Pass-Q: a bad KV shard, and a NULL output of the last Q shard's merge
    for kw, code in (({"bad_kv": 2}, cp.CP_E_SHAPE), ({"bad_o_out": True}, cp.CP_E_ARG)):
        a = _ring_arrays(N, **kw)
        st = lib.cp_ring_pass_q(N, a["q"], a["tq"], a["q_segs"], a["nq"], a["k"], a["v"], a["tk"],
                                a["kv_segs"], a["nk"], 16, 1, 128, cp.CP_BF16, 1, 0.1, a["o_parts"],
                                a["l_parts"], a["o_out"], cp.CP_F32, None, None)
        assert st == code, cp.last_error()
    # argument errors of the drivers themselves
    a = _ring_arrays(N)
    assert lib.cp_ring_pass_q(0, a["q"], a["tq"], a["q_segs"], a["nq"], a["k"], a["v"], a["tk"],
                              a["kv_segs"], a["nk"], 16, 1, 128, cp.CP_BF16, 1, 0.1, a["o_parts"],
                              a["l_parts"], a["o_out"], cp.CP_F32, None, None) == cp.CP_E_ARG
    assert lib.cp_ring_pass_kv(a["q"][0], 16, a["q_segs"][0], 1, N, N, a["k"], a["v"], a["tk"], a["kv_segs"],
                               a["nk"], 16, 1, 128, cp.CP_BF16, 1, 0.1, a["o_parts"], a["l_parts"], None,
                               None, 0x7200000, cp.CP_F32, None, None, 0, None) == cp.CP_E_ARG
    # a misaligned running-mode workspace is refused before any launch
    assert lib.cp_ring_pass_kv(a["q"][0], 16, a["q_segs"][0], 1, N, 0, a["k"], a["v"], a["tk"], a["kv_segs"],
                               a["nk"], 16, 1, 128, cp.CP_BF16, 1, 0.1, None, None, 0x7000000,
                               0x7100000, 0x7000000, cp.CP_F32, None, 0x7300008, 1 << 20,
                               None) == cp.CP_E_ARG
    assert "workspace" in cp.last_error()
    # the running-mode workspace holds one partial: O, then the LSEs at the next 256-byte boundary
    assert cp.ring_workspace_bytes(100, 16, 128) == 100 * 16 * 128 * 4 + 6400
    assert cp.ring_workspace_bytes(3, 1, 64) == 768 + 256


def test_binding_rejects_host_tensors_before_calling_the_library():
    """A host tensor's address handed to a kernel would fault the GPU: the binding refuses it (and
    strided views, wrong dtypes and shapes) before any library call. Needs no GPU."""
    import torch
    q = torch.zeros(16, 4, 64, dtype=torch.bfloat16)
    k = torch.zeros(16, 1, 64, dtype=torch.bfloat16)
    o = torch.zeros(16, 4, 64)
    lse = torch.zeros(16, 4)
    segs = [(0, 0, 16, 0)]
    with pytest.raises(ValueError, match="device tensor"):
        cp.partial_attn(q, k, k, segs, segs, True, 0.125, o, lse)
    with pytest.raises(ValueError, match="device tensor"):
        cp.merge_lse([o], [lse], o)
    with pytest.raises(ValueError, match="device tensor"):
        cp.decode_splitkv(q[:2], k, k, torch.zeros(2, dtype=torch.int64),
                          torch.zeros(2, dtype=torch.int64), 4, 0.125,
                          torch.zeros(2 * 4 * 4 * 64, dtype=torch.bfloat16), torch.zeros(2 * 4 * 4),
                          torch.zeros(2, 4, 64))
    with pytest.raises(ValueError, match="device tensor"):
        cp.ring_pass_kv(q, segs, 0, [k], [k], [segs], True, 0.125, o, o_acc=o, lse_acc=lse)


def test_binding_checks_layout_dtype_and_shape():
    """The same checks on tensors that claim to be on the device: exercised through a stand-in
    object, so no GPU is needed."""
    import torch

    class Dev:
        def __init__(self, t):
            self.t = t
            self.is_cuda = True
            self.dtype, self.shape = t.dtype, t.shape

        def is_contiguous(self):
            return self.t.is_contiguous()

        def numel(self):
            return self.t.numel()

    from context_ring_attention_amd.binding import _req
    _req(Dev(torch.zeros(4, 8)), "x", (torch.float32,), (4, 8))
    with pytest.raises(ValueError, match="contiguous"):
        _req(Dev(torch.zeros(8, 4).t()), "x")
    with pytest.raises(TypeError, match="dtype"):
        _req(Dev(torch.zeros(4, 8, dtype=torch.float16)), "x", (torch.float32,))
    with pytest.raises(ValueError, match="shape"):
        _req(Dev(torch.zeros(4, 8)), "x", None, (8, 4))
    with pytest.raises(ValueError, match="elements"):
        _req(Dev(torch.zeros(4, 8)), "x", numel=33)
    _req(12345, "raw address")   # plain integers are passed through


def test_c_program_uses_the_abi_without_python(tmp_path):
    """include/cpattn.h is valid standalone C11, and a plain C program linked against
    libcpattn.so gets the documented host-side behaviour (tests/c_abi_check.c). No GPU needed."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    lib_dir = os.path.dirname(cp.LIB_PATH)
    exe = str(tmp_path / "c_abi_check")
    src = os.path.join(ROOT, "tests", "c_abi_check.c")
    subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I",
                    os.path.join(ROOT, "include"), src, "-o", exe, "-L", lib_dir, "-lcpattn",
                    f"-Wl,-rpath,{lib_dir}"], check=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stderr
    assert res.stdout.strip() == "ok"


def test_binding_check_false_skips_only_the_tensor_checks():
    """check=False passes tensors straight to the library (for loops that validated them once);
    the library's own validation still runs and reports through CpError."""
    import torch
    q = torch.zeros(16, 6, 64, dtype=torch.bfloat16)   # 6 heads over 4 KV heads: invalid shape
    k = torch.zeros(16, 4, 64, dtype=torch.bfloat16)
    o = torch.zeros(16, 6, 64)
    lse = torch.zeros(16, 6)
    segs = [(0, 0, 16, 0)]
    with pytest.raises(ValueError, match="device tensor"):
        cp.partial_attn(q, k, k, segs, segs, True, 0.125, o, lse)
    with pytest.raises(cp.CpError, match="CP_E_SHAPE"):
        cp.partial_attn(q, k, k, segs, segs, True, 0.125, o, lse, stream=0, check=False)


def test_product_and_oracle_share_no_code():
    """The HIP path never imports, includes or loads the oracle, and the oracle never refers to
    the HIP path except in its header comments (which say it does not)."""
    import glob
    prod = [f for ext in ("py", "hip", "cpp", "h") for f in
            glob.glob(os.path.join(ROOT, "context_ring_attention_amd", "**", f"*.{ext}"), recursive=True)]
    prod += glob.glob(os.path.join(ROOT, "include", "*.h"))
    assert prod
    for f in prod:
        text = open(f).read()
        assert not re.search(r"\bimport\s+oracle|\bfrom\s+oracle\b|#include\s*[<\"][^>\"]*oracle|liboracle",
                             text), f
    for f in glob.glob(os.path.join(ROOT, "oracle", "*.[ch]")) + glob.glob(os.path.join(ROOT, "oracle", "*.py")):
        code = re.sub(r"/\*.*?\*/", "", open(f).read(), flags=re.S)       # C comments
        code = re.sub(r'""".*?"""', "", code, flags=re.S)                   # Python docstrings
        code = "\n".join(l.split("#", 1)[0] if f.endswith(".py") else l for l in code.splitlines())
        assert "context_ring_attention_amd" not in code and "cpattn" not in code, f


def test_bench_uses_the_oracle_only_for_its_cpu_baseline():
    import ast
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    users = set()
    for fn in ast.walk(tree):
        if isinstance(fn, ast.FunctionDef):
            for node in ast.walk(fn):
                if isinstance(node, ast.Import) and any(a.name == "oracle" for a in node.names):
                    users.add(fn.name)
                if isinstance(node, ast.ImportFrom) and node.module == "oracle":
                    users.add(fn.name)
    top = [n for n in tree.body if isinstance(n, (ast.Import, ast.ImportFrom))
           and ("oracle" in [a.name for a in n.names] or getattr(n, "module", None) == "oracle")]
    assert not top and users == {"run_cpu_baseline"}, (top, users)


def test_binding_fails_loudly_without_the_library():
    """No silent fallback: with libcpattn.so absent, loading (and so every entry point) raises."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("cpattn_binding_copy", cp.__file__)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.LIB_PATH = os.path.join(ROOT, "no_such_dir", "libcpattn.so")
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        mod.load()
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        mod.shard_map([(0, 0, 16)], 2, 0)


def test_c_abi_host_code_under_address_sanitizer(tmp_path):
    """The C ABI's host code (api.cpp) built with AddressSanitizer, the kernel launchers replaced
    by stubs that abort, driven by tests/c_abi_check.c: shard map, validation and selector paths
    must run without any ASan report. Host code only; no device code is built."""
    import shutil
    import subprocess
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    csrc = os.path.join(ROOT, "context_ring_attention_amd", "csrc")
    lib = str(tmp_path / "libcpattn.so")
    san = ["-Xarch_host", "-fsanitize=address", "-fno-omit-frame-pointer", "-g"]
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc)))
    subprocess.run([hipcc, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
                    "-std=c++17", "-O1", "-fPIC", "-shared", *san,
                    "-I", os.path.join(ROOT, "include"), "-I", csrc,
                    os.path.join(csrc, "api.cpp"), os.path.join(ROOT, "tests", "host_launch_stubs.cpp"),
                    "-o", lib], check=True, capture_output=True)
    exe = str(tmp_path / "c_abi_check_asan")
    clang = os.path.join(rocm, "llvm", "bin", "clang")   # the same sanitizer runtime as the library
    if not os.path.exists(clang):
        pytest.skip("ROCm clang not available")
    subprocess.run([clang, "-std=c11", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_check.c"),
                    "-o", exe, "-L", str(tmp_path), "-lcpattn", f"-Wl,-rpath,{tmp_path}"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert res.returncode == 0 and "ERROR: AddressSanitizer" not in res.stderr, res.stderr[-2000:]
    assert res.stdout.strip() == "ok"
