"""The C-ABI library loads on the host and exports every entry point that
include/kda.h declares; metadata errors are reported without touching a GPU
(each failing call returns before any HIP runtime call).  The partition
query only asks the HIP runtime for the device's compute-unit count."""

import ctypes
import functools
import os
import re

import pytest

import kda_gated_delta_amd as kda

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "kda.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("kda_chunk_prefill", "kda_chunk_prefill_split", "kda_chunk_prefill_fused",
              "kda_chunk_prefill_partition", "kda_chunk_prefill_workspace_size", "kda_decode",
              "kda_qk_l2norm",
              "kda_packed_decode", "kda_state_to_pool", "kda_status_string",
              "kda_chunk_backward", "kda_chunk_backward_workspace_size"):
        assert n in names
    assert set(names) == set(kda.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(kda.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_build_id_matches_sources():
    """The loaded library carries the hash of the sources it was built
    from; it must be this tree's."""
    assert kda.check_build_matches_sources() == kda.build_id()
    assert len(kda.build_id()) == 32


def test_status_strings():
    lib = kda.load()
    for code in range(7):
        assert lib.kda_status_string(code).startswith(b"KDA_")
    assert b"unknown" in lib.kda_status_string(99)


NULL = ctypes.c_void_p(0)
FAKE = ctypes.c_void_p(0x1000)       # never dereferenced: every call below fails its checks first
MISALIGNED = ctypes.c_void_p(0x1008)


def test_l2norm_metadata_errors():
    lib = kda.load()
    assert lib.kda_qk_l2norm(FAKE, FAKE, 0, 128, NULL) == 0          # nothing to do
    assert lib.kda_qk_l2norm(FAKE, FAKE, -1, 128, NULL) == 2
    assert lib.kda_qk_l2norm(FAKE, FAKE, 4, 64, NULL) == 3
    assert lib.kda_qk_l2norm(NULL, FAKE, 4, 128, NULL) == 1
    assert lib.kda_qk_l2norm(MISALIGNED, FAKE, 4, 128, NULL) == 4


def _prefill(lib, entry="kda_chunk_prefill", **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, s0=NULL, cu=NULL, n=0,
             B=1, T=64, H=1, HV=1, K=128, V=128, o=FAKE, fs=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return getattr(lib, entry)(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["cu"], a["n"],
                               a["B"], a["T"], a["H"], a["HV"], a["K"], a["V"], a["o"], a["fs"],
                               a["ws"], a["wsb"], NULL)


@pytest.mark.parametrize("entry", ["kda_chunk_prefill", "kda_chunk_prefill_split"])
def test_prefill_metadata_errors(entry):
    lib = kda.load()
    _prefill = functools.partial(globals()["_prefill"], entry=entry)
    assert _prefill(lib, q=NULL) == 1
    assert _prefill(lib, fs=NULL) == 1
    assert _prefill(lib, H=3, HV=4) == 2
    assert _prefill(lib, B=0) == 2
    assert _prefill(lib, T=-1) == 2
    assert _prefill(lib, K=64) == 3
    assert _prefill(lib, V=256) == 3
    assert _prefill(lib, cu=FAKE, n=2, B=2) == 2          # packed sequences need B == 1
    assert _prefill(lib, cu=FAKE, n=0) == 2
    assert _prefill(lib, v=MISALIGNED) == 4
    assert _prefill(lib, ws=NULL) == 1
    assert _prefill(lib, wsb=1000) == 5                    # KDA_ERR_WORKSPACE
    # the smallest workspace is one 66048-byte chunk slot per value head,
    # whatever the unit count (so the errors do not depend on the partition)
    assert kda.PREFILL_SLOT_BYTES == 66048
    assert _prefill(lib, H=2, HV=4, wsb=4 * 66048 - 16) == 5
    # value heads are bounded (32-bit offsets within a chunk)
    assert _prefill(lib, H=1, HV=65536) == 2
    assert _prefill(lib, H=65536, HV=65536) == 2
    assert _prefill(lib, B=64, H=64, HV=64, wsb=64 * 66048 - 16) == 5


def test_partition_query():
    """kda_chunk_prefill runs the fused form from 3/4 as many (sequence,
    value head) units as compute units; without a device the query takes
    MI355X's 256, which is also the count on the MI355X."""
    lib = kda.load()
    assert lib.kda_chunk_prefill_partition(1, 96, 0) == 0           # 96 units: split
    assert lib.kda_chunk_prefill_partition(1, 191, 0) == 0
    assert lib.kda_chunk_prefill_partition(1, 192, 0) == 1          # 192 = 3/4 of 256: fused
    assert lib.kda_chunk_prefill_partition(16, 64, 0) == 1
    assert lib.kda_chunk_prefill_partition(1, 32, 16) == 1          # 16 packed sequences x 32 heads
    assert lib.kda_chunk_prefill_partition(1, 32, 5) == 0
    assert lib.kda_chunk_prefill_partition(0, 32, 0) == -2
    assert lib.kda_chunk_prefill_partition(1, 0, 0) == -2
    assert lib.kda_chunk_prefill_partition(1, 65536, 0) == -2
    assert kda.prefill_partition(1, 96) == "split" and kda.prefill_partition(4, 64) == "fused"


def test_workspace_size_formula():
    lib = kda.load()
    slot = 66048
    # one window of chunk slots per value head: the window holds
    # min(floor(B*T/64) + N + 1, floor(2 GiB / (HV * slot))) slots; when it
    # holds them all, 4 bytes per slot and value head of ready flags follow
    # and one status word per (sequence, value head) (rounded up to 256 bytes)
    flags = lambda n: (n * 4 + 255) // 256 * 256
    assert lib.kda_chunk_prefill_workspace_size(1, 8192, 96, 96, 128, 128, 0) == 130 * 96 * slot + flags(131 * 96)
    assert lib.kda_chunk_prefill_workspace_size(1, 65536, 96, 96, 128, 128, 0) == (2**31 // (96 * slot)) * 96 * slot
    assert lib.kda_chunk_prefill_workspace_size(2, 1000, 8, 8, 128, 128, 0) == 34 * 8 * slot + flags(36 * 8)
    assert lib.kda_chunk_prefill_workspace_size(1, 500, 2, 4, 128, 128, 5) == 13 * 4 * slot + flags(18 * 4)
    assert lib.kda_chunk_prefill_workspace_size(1, 64, 1, 1, 64, 128, 0) == 0


def _decode(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, pool=FAKE, stride=12 * 128 * 128, n=8,
             idx=FAKE, B=4, H=12, HV=12, K=128, V=128, o=FAKE)
    a.update(kw)
    return lib.kda_decode(a["q"], a["k"], a["v"], a["g"], a["beta"], a["pool"], a["stride"], a["n"],
                          a["idx"], a["B"], a["H"], a["HV"], a["K"], a["V"], a["o"], NULL)


def test_decode_metadata_errors():
    lib = kda.load()
    assert _decode(lib, B=0) == 0
    assert _decode(lib, idx=NULL) == 1
    assert _decode(lib, H=5) == 2
    assert _decode(lib, stride=100) == 2
    assert _decode(lib, stride=12 * 128 * 128 + 4) == 4
    assert _decode(lib, K=64) == 3
    assert _decode(lib, o=MISALIGNED) == 4


def _to_pool(lib, **kw):
    a = dict(state=FAKE, N=4, HV=12, K=128, V=128, pool=FAKE, stride=12 * 128 * 128, n=8, idx=FAKE)
    a.update(kw)
    return lib.kda_state_to_pool(a["state"], a["N"], a["HV"], a["K"], a["V"], a["pool"], a["stride"],
                                 a["n"], a["idx"], NULL)


def test_state_to_pool_metadata_errors():
    lib = kda.load()
    assert _to_pool(lib, N=0) == 0
    assert _to_pool(lib, N=-1) == 2
    assert _to_pool(lib, HV=0) == 2
    assert _to_pool(lib, n=-1) == 2
    assert _to_pool(lib, K=64) == 3
    assert _to_pool(lib, state=NULL) == 1
    assert _to_pool(lib, idx=NULL) == 1
    assert _to_pool(lib, pool=NULL) == 1
    assert _to_pool(lib, stride=100) == 2
    assert _to_pool(lib, stride=12 * 128 * 128 + 4) == 4
    assert _to_pool(lib, state=MISALIGNED) == 4
    assert _to_pool(lib, pool=MISALIGNED) == 4


def _packed(lib, **kw):
    a = dict(qkv=FAKE, rs=3 * 12 * 128, rg=FAKE, rb=FAKE, al=FAKE, dt=FAKE, pool=FAKE,
             stride=12 * 128 * 128, n=8, idx=FAKE, B=4, H=12, K=128, V=128, o=FAKE)
    a.update(kw)
    return lib.kda_packed_decode(a["qkv"], a["rs"], a["rg"], a["rb"], a["al"], a["dt"], a["pool"], a["stride"],
                                 a["n"], a["idx"], a["B"], a["H"], a["K"], a["V"], a["o"], NULL)


def test_packed_decode_metadata_errors():
    lib = kda.load()
    assert _packed(lib, B=0) == 0
    assert _packed(lib, B=-1) == 2
    assert _packed(lib, H=0) == 2
    assert _packed(lib, K=64) == 3
    assert _packed(lib, qkv=NULL) == 1
    assert _packed(lib, al=NULL) == 1
    assert _packed(lib, dt=NULL) == 1
    assert _packed(lib, pool=NULL) == 1
    assert _packed(lib, rs=3 * 12 * 128 - 8) == 2
    assert _packed(lib, rs=3 * 12 * 128 + 4) == 4
    assert _packed(lib, stride=100) == 2
    assert _packed(lib, qkv=MISALIGNED) == 4
    assert _packed(lib, o=MISALIGNED) == 4


def test_fused_prefill_metadata_errors():
    lib = kda.load()

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, s0=NULL, cu=NULL, n=0,
                 B=1, T=64, H=1, HV=1, K=128, V=128, o=FAKE, fs=FAKE)
        a.update(kw)
        return lib.kda_chunk_prefill_fused(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["cu"], a["n"],
                                           a["B"], a["T"], a["H"], a["HV"], a["K"], a["V"], a["o"], a["fs"], NULL)
    assert call(q=NULL) == 1
    assert call(fs=NULL) == 1
    assert call(H=3, HV=4) == 2
    assert call(B=0) == 2
    assert call(K=64) == 3
    assert call(cu=FAKE, n=2, B=2) == 2
    assert call(H=1, HV=65536) == 2
    assert call(v=MISALIGNED) == 4


def _backward(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, s0=NULL, cu=NULL, n=0,
             B=1, T=64, H=1, HV=1, K=128, V=128, do=FAKE, dht=NULL, dq=FAKE, dk=FAKE, dv=FAKE,
             dg=FAKE, db=FAKE, dh0=NULL, gd=1, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.kda_chunk_backward(a["q"], a["k"], a["v"], a["g"], a["beta"], a["s0"], a["cu"], a["n"],
                                  a["B"], a["T"], a["H"], a["HV"], a["K"], a["V"], a["do"], a["dht"],
                                  a["dq"], a["dk"], a["dv"], a["dg"], a["db"], a["dh0"], a["gd"], a["ws"], a["wsb"],
                                  NULL)


def test_backward_metadata_errors():
    lib = kda.load()
    assert _backward(lib, q=NULL) == 1
    assert _backward(lib, do=NULL) == 1
    assert _backward(lib, dg=NULL) == 1
    assert _backward(lib, H=3, HV=4) == 2
    assert _backward(lib, B=0) == 2
    assert _backward(lib, T=-1) == 2
    assert _backward(lib, K=64) == 3
    assert _backward(lib, cu=FAKE, n=2, B=2) == 2
    assert _backward(lib, dv=MISALIGNED) == 4
    assert _backward(lib, ws=NULL) == 1
    assert _backward(lib, wsb=1000) == 5
    assert _backward(lib, gd=2) == 3                        # unknown gradient dtype
    assert _backward(lib, gd=-1) == 3
    assert _backward(lib, H=1, HV=65536) == 2          # value heads are a grid dimension


def test_backward_workspace_size_formula():
    lib = kda.load()
    rec = 139392 * 4     # record per chunk slot (float32, q^ and k^ as bf16)
    # floor(B*T/64) + N + 1 slots per value head, plus two float32 [tokens, HV, 128] buffers
    assert lib.kda_chunk_backward_workspace_size(1, 8192, 96, 96, 128, 128, 0) == \
        (128 + 1 + 1) * 96 * rec + 8192 * 96 * 128 * 4 * 2
    assert lib.kda_chunk_backward_workspace_size(1, 500, 2, 4, 128, 128, 5) == \
        (7 + 5 + 1) * 4 * rec + 500 * 4 * 128 * 4 * 2
    assert lib.kda_chunk_backward_workspace_size(1, 64, 1, 1, 64, 128, 0) == 0


def test_noalloc_rejects_sizes_beyond_its_static_workspace():
    """kda_chunk_prefill_noalloc runs in windows of as many chunk slots as its
    64 MiB static workspace holds, so it takes any length; only more value
    heads than one slot each fits (HV > 1016) returns KDA_ERR_WORKSPACE (5),
    checked before the device is touched.  Metadata errors come first."""
    lib = kda.load()
    call = lambda **kw: lib.kda_chunk_prefill_noalloc(
        FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, 0, kw.get("B", 1), kw.get("T", 64), kw.get("H", 1),
        kw.get("HV", 1), kw.get("K", 128), 128, FAKE, FAKE, NULL)
    assert 1016 * 66048 <= kda.NOALLOC_WORKSPACE_BYTES < 1017 * 66048
    assert call(H=1017, HV=1017) == 5
    assert call(H=8, HV=2048, T=1) == 5
    assert call(K=64) == 3
    assert call(H=3, HV=4) == 2
