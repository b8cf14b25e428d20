"""Argument checks of the C ABI, on a machine with no GPU.

Validation is pure host code that runs before any HIP call, so every bad
argument below is reported with its status code here, and nothing is
enqueued.  Data pointers are fake (never dereferenced on the host).  Also
checks that libra.so exports every function include/ra.h declares.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

RA_OK, RA_E_INVALID, RA_E_UNSUPPORTED, RA_E_ALIGN, RA_E_HIP, RA_E_WORKSPACE = range(6)
FAKE = 0x10000000  # 16-byte aligned, never dereferenced


def _L():
    from ring_blockwise_softmax_amd import _lib
    return _lib


def T(b, s, h, d, dtype=0, data=FAKE, strides=None):
    L = _L()
    if strides is None:
        strides = (s * h * d, h * d, d)
    return L.RaTensor(data, dtype, 0, b, s, h, d, *strides)


def LSE(b, s, h, data=FAKE, dtype=1):
    L = _L()
    return L.RaTensor(data, dtype, 0, b, s, h, 1, h * s, 1, s)


def attn(q, k, v, mask, out, lse):
    L = _L()
    return L.lib().ra_block_attn_fwd(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), mask,
                                     ctypes.byref(out), ctypes.byref(lse), None, 0, None)


def good(d=128, dtype=0, Sq=64, Sk=64, Hq=4, Hkv=2):
    return (T(1, Sq, Hq, d, dtype), T(1, Sk, Hkv, d, dtype), T(1, Sk, Hkv, d, dtype),
            T(1, Sq, Hq, d, 1), LSE(1, Sq, Hq))


def test_exports_match_header():
    L = _L()
    lib = L.lib()
    with open(os.path.join(ROOT, "include", "ra.h")) as f:
        text = f.read()
    declared = set(re.findall(r"^[A-Za-z_][\w \*]*?\b(ra_\w+)\s*\(", text, flags=re.M))
    assert {"ra_block_attn_fwd", "ra_merge", "ra_ring_forward", "ra_ring_plan"} <= declared
    for name in declared:
        assert hasattr(lib, name), f"libra.so does not export {name}"
    assert declared <= set(L.EXPORTS), "binding is missing a declared entry point"
    assert lib.ra_version() == 1


def test_status_strings():
    lib = _L().lib()
    assert lib.ra_status_str(0) == b"RA_OK"
    assert lib.ra_status_str(5) == b"RA_E_WORKSPACE"


@pytest.mark.parametrize("mutate,status", [
    (lambda a: a[0].__setattr__("dtype", 7), RA_E_UNSUPPORTED),         # unknown dtype
    (lambda a: [t.__setattr__("d", 96) for t in a[:3]], RA_E_UNSUPPORTED),  # head_dim 96
    (lambda a: a[1].__setattr__("h", 3) or a[2].__setattr__("h", 3), RA_E_INVALID),  # Hq % Hkv
    (lambda a: a[0].__setattr__("data", None), RA_E_INVALID),           # null pointer
    (lambda a: a[0].__setattr__("data", FAKE + 2), RA_E_ALIGN),         # misaligned
    (lambda a: a[1].__setattr__("ss", 260), RA_E_ALIGN),                 # stride not 16 B
    (lambda a: a[1].__setattr__("dtype", 1), RA_E_INVALID),             # mixed dtypes
    (lambda a: a[3].__setattr__("dtype", 0), RA_E_UNSUPPORTED),         # bf16 out
    (lambda a: a[3].__setattr__("s", 63), RA_E_INVALID),                 # out shape
    (lambda a: a[4].__setattr__("h", 2), RA_E_INVALID),                  # lse shape
    (lambda a: a[4].__setattr__("data", FAKE + 2), RA_E_ALIGN),         # lse alignment
    (lambda a: a[2].__setattr__("s", 32), RA_E_INVALID),                 # k/v length differ
    (lambda a: a[1].__setattr__("b", 2), RA_E_INVALID),                  # batch mismatch
    (lambda a: a[0].__setattr__("sh", 1 << 33), RA_E_UNSUPPORTED),        # head stride > int32
    (lambda a: a[2].__setattr__("ss", 72 << 20), RA_E_UNSUPPORTED),       # bf16 V token stride: 32-bit tile offsets
])
def test_block_attn_rejects(mutate, status):
    args = list(good())
    mutate(args)
    q, k, v, out, lse = args
    assert attn(q, k, v, 0, out, lse) == status
    assert _L().lib().ra_last_error()


def test_work_tile_count_limit():
    """B x Hq x Sq beyond a launch's 32-bit work-tile count is refused on the
    host (the descriptors are never dereferenced, so no memory is needed)."""
    q, k, v, out, lse = good()
    for t in (q, k, v, out):
        t.b = 4096
    lse.b = 4096
    for t in (q, out):
        t.s = 1 << 20
        t.h = 1024
    lse.s, lse.h = 1 << 20, 1024
    k.h = v.h = 1024
    assert attn(q, k, v, 0, out, lse) == RA_E_UNSUPPORTED
    assert "work-tile" in _L().lib().ra_last_error().decode()


def test_bf16_kv_token_stride_limit():
    """The largest accepted bf16 K/V token stride keeps (31 * ss + d) * 2 bytes
    within 32 bits; one element more (rounded to a 16-byte multiple) is refused.
    fp32 K/V address in 64 bits and take the larger stride.  Each call carries
    an unknown mask kind, which is checked after the tensors, so a stride that
    passes shows up as the mask error and nothing is ever enqueued."""
    d = 128
    lim = (2**31 - 1 - d) // 31
    ok = lim - lim % 8
    assert (31 * ok + d) * 2 < 2**32 and 31 * ok + d <= 2**31 - 1
    for dtype, ss, want in ((0, ok, "mask"), (0, ok + 8, "token stride"), (1, ok + 8, "mask")):
        q, k, v, out, lse = good(d=d, dtype=dtype)
        k.ss = ss
        st = attn(q, k, v, 3, out, lse)
        msg = _L().lib().ra_last_error().decode()
        assert want in msg, (dtype, ss, st, msg)
        assert st == (RA_E_INVALID if want == "mask" else RA_E_UNSUPPORTED)


def test_block_attn_rejects_mask():
    q, k, v, out, lse = good()
    assert attn(q, k, v, 3, out, lse) == RA_E_INVALID
    q, k, v, out, lse = good(Sq=80, Sk=64)
    assert attn(q, k, v, 2, out, lse) == RA_E_INVALID   # bottom-right needs Sq <= Sk


def test_empty_query_block_is_a_noop():
    q, k, v, out, lse = good(Sq=0)
    q.data = out.data = lse.data = None
    assert attn(q, k, v, 0, out, lse) == RA_OK


def _ring(q, k, v, P, kind, fuse, out, lse, ws=None, ws_bytes=0, rank=-1):
    L = _L()
    lay = L.RaLayout(kind, 0, rank, fuse, ws, ws_bytes)
    return L.lib().ra_ring_forward(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), P, ctypes.byref(lay),
                                   ctypes.byref(out), ctypes.byref(lse), None)


def test_ring_rejects():
    q, k, v, out, lse = good(Sq=96, Sk=96)
    assert _ring(q, k, v, 5, 0, 1, out, lse) == RA_E_INVALID        # 96 % 5
    assert _ring(q, k, v, 5, 2, 1, out, lse) == RA_E_INVALID        # 96 % 10
    assert _ring(q, k, v, 0, 0, 1, out, lse) == RA_E_UNSUPPORTED
    assert _ring(q, k, v, 17, 0, 1, out, lse) == RA_E_UNSUPPORTED
    assert _ring(q, k, v, 4, 9, 1, out, lse) == RA_E_INVALID        # layout kind
    assert _ring(q, k, v, 4, 0, 1, out, lse, rank=4) == RA_E_INVALID
    # unfused needs workspace; too small or missing is reported, nothing runs
    assert _ring(q, k, v, 4, 0, 0, out, lse) == RA_E_WORKSPACE
    assert _ring(q, k, v, 4, 0, 0, out, lse, ws=FAKE, ws_bytes=100) == RA_E_WORKSPACE
    q2, k2, v2, out2, lse2 = good(Sq=1, Sk=96)
    assert _ring(q2, k2, v2, 4, 0, 1, out2, lse2) == RA_E_INVALID   # Sq != Sk for a ring layout
    q3, k3, v3, out3, lse3 = good(Sq=96, Sk=64)
    assert _ring(q3, k3, v3, 4, 4, 1, out3, lse3) == RA_E_INVALID   # causal K/V-sharded: Sq > Sk
    assert _ring(q3, k3, v3, 4, 5, 1, out3, lse3) == RA_E_INVALID   # no such layout kind


def test_workspace_queries():
    L = _L()
    lib = L.lib()
    q, k, v, out, lse = good(Sq=24000, Sk=24000, Hq=32, Hkv=32)
    fused = L.RaLayout(0, 0, -1, 1, None, 0)
    unfused = L.RaLayout(0, 0, -1, 0, None, 0)
    assert lib.ra_ring_workspace_bytes(ctypes.byref(q), ctypes.byref(k), 4, ctypes.byref(fused)) == 0
    n = lib.ra_ring_workspace_bytes(ctypes.byref(q), ctypes.byref(k), 4, ctypes.byref(unfused))
    assert n >= 24000 * 32 * 129 * 4
    # decode shape: split-K partials need scratch
    q = T(16, 1, 32, 128)
    k = T(16, 262144, 1, 128)
    assert lib.ra_block_attn_workspace_bytes(ctypes.byref(q), ctypes.byref(k)) > 0
    # fused KV-sharded decode gathers every block's sub-block partials at once:
    # 16 query tiles need 32 partials per row to cover the chip twice, i.e. 4
    # sub-blocks of 8192 keys in each of the 8 blocks
    kvs = L.RaLayout(3, 0, -1, 1, None, 0)
    n = lib.ra_ring_workspace_bytes(ctypes.byref(q), ctypes.byref(k), 8, ctypes.byref(kvs))
    assert n == 8 * 4 * 16 * 32 * 1 * (128 + 1) * 4
    # a 4096-token prefill chunk at the end of a 131072-token cache over 8 shards:
    # 1024 query tiles per block is under two rounds of work-groups, so all 8
    # blocks' partials are gathered (one partial per block and row)
    q = T(1, 4096, 32, 128)
    k = T(1, 131072, 8, 128)
    kvc = L.RaLayout(4, 0, -1, 1, None, 0)
    n = lib.ra_ring_workspace_bytes(ctypes.byref(q), ctypes.byref(k), 8, ctypes.byref(kvc))
    assert n == 8 * 1 * 1 * 32 * 4096 * (128 + 1) * 4


def test_merge_rejects():
    L = _L()
    lib = L.lib()
    out, bout = T(1, 10, 2, 128, 1), T(1, 10, 2, 128, 1, data=FAKE + 0x100000)
    lse, blse = LSE(1, 10, 2), LSE(1, 10, 2, data=FAKE + 0x200000)
    bad = T(1, 11, 2, 128, 1, data=FAKE + 0x100000)
    assert lib.ra_merge(ctypes.byref(out), ctypes.byref(lse), ctypes.byref(bad), ctypes.byref(blse), None) == RA_E_INVALID
    assert lib.ra_merge(ctypes.byref(out), ctypes.byref(lse), ctypes.byref(out), ctypes.byref(blse), None) == RA_E_INVALID
    b16 = T(1, 10, 2, 128, 0, data=FAKE + 0x100000)
    assert lib.ra_merge(ctypes.byref(out), ctypes.byref(lse), ctypes.byref(b16), ctypes.byref(blse), None) == RA_E_UNSUPPORTED


@pytest.mark.parametrize("d", [12, 96, 192, 512])
def test_merge_rejects_head_dims_that_split_a_row_over_waves(d):
    """A row's d/4 threads must sit in one wave (the lse is rewritten by one of
    them after all have read it), so d/4 must divide 64."""
    L = _L()
    lib = L.lib()
    out, bout = T(1, 10, 2, d, 1), T(1, 10, 2, d, 1, data=FAKE + 0x100000)
    lse, blse = LSE(1, 10, 2), LSE(1, 10, 2, data=FAKE + 0x200000)
    st = lib.ra_merge(ctypes.byref(out), ctypes.byref(lse), ctypes.byref(bout), ctypes.byref(blse), None)
    assert st == RA_E_UNSUPPORTED
    assert b"head_dim" in lib.ra_last_error()


def test_probe_library_rejects_bad_arguments():
    """The benchmark's MFMA probe library loads and checks its arguments on
    the host (nothing is launched)."""
    lib = ctypes.CDLL(os.path.join(ROOT, "ring_blockwise_softmax_amd", "libra_probe.so"))
    assert lib.ra_probe_mfma_loop(0, None, None, 0, 1, None) != 0     # no grid
    assert lib.ra_probe_mfma_loop(0, None, ctypes.c_void_p(FAKE), 8, 1, None) != 0  # operands missing


def test_noalloc_rejects_before_any_hip_call():
    """The no-allocation entry point checks its arguments and the size of the
    split partials it would need on the host: bad arguments and blocks whose
    partials exceed the static scratch are rejected with nothing enqueued."""
    L = _L()
    lib = L.lib()

    def call(q, k, v, mask, o, l):
        return lib.ra_block_attn_fwd_noalloc(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), mask,
                                             ctypes.byref(o), ctypes.byref(l), None)

    q, k, v, o, l = good()
    q.dtype = 7
    assert call(q, k, v, 0, o, l) == RA_E_UNSUPPORTED
    q, k, v, o, l = good()
    assert call(q, k, v, 9, o, l) == RA_E_INVALID
    # B1 Hq32/Hkv1 Sq4 against 32768 keys: 4 x 32 packed rows in one tile, so
    # the keys are split 512 ways: 512 * 32 * 4 * (128 + 1) * 4 bytes of
    # partials, just over the 32 MiB scratch.
    q, k, v, o, l = good(Sq=4, Sk=32768, Hq=32, Hkv=1)
    need = lib.ra_block_attn_workspace_bytes(ctypes.byref(q), ctypes.byref(k))
    assert need == 512 * 32 * 4 * 129 * 4 > L.NOALLOC_SCRATCH_BYTES
    assert call(q, k, v, 0, o, l) == RA_E_UNSUPPORTED
    assert b"static scratch" in lib.ra_last_error()


@pytest.mark.parametrize("entry", ["block_attn_fwd", "merge", "ring_forward", "noalloc"])
def test_python_entry_points_refuse_host_tensors(entry):
    """Host tensors would hand host pointers to the kernels: the binding
    refuses them before calling the library."""
    import torch
    import ring_blockwise_softmax_amd as ra
    q = torch.zeros(1, 64, 2, 64, dtype=torch.bfloat16)
    out = torch.zeros(1, 64, 2, 64)
    lse = torch.zeros(1, 2, 64)
    with pytest.raises(ValueError, match="GPU"):
        if entry == "block_attn_fwd":
            ra.block_attn_fwd(q, q, q)
        elif entry == "merge":
            ra.merge(out, lse, out.clone(), lse.clone())
        elif entry == "ring_forward":
            ra.ring_forward(q, q, q, 2)
        else:
            ra.block_attn_fwd_noalloc(q, q, q, out, lse)


def test_last_error_is_thread_local():
    """Each host thread reads back the message of its own last failure, even
    when several threads fail differently at the same time."""
    import threading
    lib = _L().lib()
    barrier = threading.Barrier(4)
    seen = {}

    def worker(i):
        q, k, v, out, lse = good()
        if i == 0:
            q.dtype = 7                      # unknown dtype
            want = "unknown dtype"
        elif i == 1:
            k.h = v.h = 3                    # Hq % Hkv
            want = "multiple of Hkv"
        elif i == 2:
            out.s = 63                       # out shape
            want = "out shape"
        else:
            want = "unknown mask kind"
        barrier.wait()
        msgs = []
        for _ in range(200):
            st = attn(q, k, v, 3 if i == 3 else 0, out, lse)
            assert st != RA_OK
            msgs.append(lib.ra_last_error().decode())
        seen[i] = (want, msgs)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    for i, (want, msgs) in seen.items():
        assert all(want in m for m in msgs), (i, want, [m for m in msgs if want not in m][:3])
