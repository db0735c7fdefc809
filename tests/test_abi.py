"""The C-ABI library on the CPU: it loads, exports every declared entry point, plans
workspace as documented and rejects host-visible argument errors before launching
anything.  None of these calls reaches a kernel, so no GPU is needed."""

import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
           if f.endswith(".h")]


@pytest.fixture(scope="module")
def pk():
    import paged_kv_cache_351_amd as pk
    if not os.path.exists(pk.LIB_PATH):
        from paged_kv_cache_351_amd.build import build
        build(verbose=False)
    pk.lib()
    return pk


def declared_functions():
    names = []
    for h in HEADERS:
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(pa_[a-z0-9_]+)\s*\(",
                            src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["pa_decode", "pa_write_kv", "pa_copy_blocks", "pa_decode_workspace_size",
              "pa_last_error", "pa_version"]:
        assert n in names


def test_library_exports_every_declared_symbol(pk):
    L = ctypes.CDLL(pk.LIB_PATH)
    for n in declared_functions():
        assert hasattr(L, n), n


def test_binding_names_match_the_abi(pk):
    for n in ["pa_decode", "pa_decode_cached", "pa_decode_append", "pa_write_kv", "pa_copy_blocks",
              "pa_decode_workspace_size", "pa_last_error", "pa_version"]:
        assert callable(getattr(pk, n))


def test_version(pk):
    assert pk.pa_version() == 9


@pytest.mark.parametrize("N,H,HKV,D,L", [(256, 32, 8, 128, 4096), (32, 64, 8, 128, 32768),
                                         (4, 4, 4, 64, 41), (64, 32, 32, 128, 2048), (3, 8, 2, 64, 0),
                                         (1, 8, 8, 128, 1)])
def test_workspace_size_formula(pk, N, H, HKV, D, L):
    # waves: one per 8 tiles of the longest possible batch, at least 1, at most 2048;
    # up to five chunks per wave (a head and four tail parts); a 256-byte header and
    # 16 bytes per chunk, then two partial slots of (D + 2) floats per query head of
    # the group per chunk, each region 256-byte aligned
    up = lambda x: -(-x // 256) * 256
    waves = min(2048, max(1, -(-(N * HKV * math.ceil(L / 16)) // 8)))
    chunks, g = 5 * waves, H // HKV
    got = pk.pa_decode_workspace_size(N, H, HKV, D, L)
    assert got == up(256 + chunks * 16) + up(2 * chunks * g * 2 * 4) + 2 * chunks * g * D * 4


def test_workspace_size_rejects_bad_arguments(pk):
    assert pk.pa_decode_workspace_size(-1, 8, 2, 128, 100) == 0
    assert pk.pa_decode_workspace_size(4, 8, 3, 128, 100) == 0
    assert pk.pa_decode_workspace_size(4, 8, 2, 128, -1) == 0
    assert pk.pa_decode_workspace_size(4, 8, 2, 128, (1 << 24) + 1) == 0


FAKE = 1 << 20  # a 16-byte aligned, non-null address that is never dereferenced


def call_decode(pk, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE, N=4, H=8, HKV=2, D=128, BS=16, NB=100,
             MB=10, L=160, scale=0.088, dt=2, out=FAKE, ws=FAKE, wsb=0, stream=None)
    a.update(over)
    return pk.lib().pa_decode(a["q"], a["k"], a["v"], a["bt"], a["lens"], a["N"], a["H"], a["HKV"],
                              a["D"], a["BS"], a["NB"], a["MB"], a["L"], a["scale"], a["dt"],
                              a["out"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("over,status,words", [
    (dict(D=96), 2, "head_dim"),
    (dict(BS=12), 2, "block_size"),
    (dict(H=9), 1, "multiple"),
    (dict(H=34, HKV=1), 2, "at most 16"),
    (dict(dt=7), 1, "dtype"),
    (dict(L=161), 1, "max_seq_len"),
    (dict(NB=0), 1, "num_blocks"),
    (dict(q=None), 1, "null"),
    (dict(out=FAKE + 4), 1, "aligned"),
    (dict(scale=float("nan")), 1, "finite"),
    (dict(L=1000, MB=100, wsb=16), 3, "workspace"),
    (dict(L=1000, MB=100, ws=None, wsb=1 << 30), 3, "workspace"),
    (dict(wsb=1 << 30, ws=FAKE + 16), 3, "256-byte"),
    (dict(L=(1 << 24) + 16, MB=1 << 21), 2, "above"),
])
def test_decode_rejects_host_visible_errors(pk, over, status, words):
    assert call_decode(pk, **over) == status
    assert words in pk.pa_last_error()


def test_decode_with_no_sequences_is_a_no_op(pk):
    assert call_decode(pk, N=0, q=None, out=None) == 0


@pytest.mark.parametrize("over,status,words", [
    (dict(D=96), 2, "head_dim"),
    (dict(q=None), 1, "null"),
    (dict(L=1000, MB=100, wsb=16), 3, "workspace"),
])
def test_decode_cached_rejects_host_visible_errors(pk, over, status, words):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE, N=4, H=8, HKV=2, D=128, BS=16, NB=100,
             MB=10, L=160, scale=0.088, dt=2, out=FAKE, ws=FAKE, wsb=0, stream=None)
    a.update(over)
    assert pk.lib().pa_decode_cached(a["q"], a["k"], a["v"], a["bt"], a["lens"], a["N"], a["H"],
                                     a["HKV"], a["D"], a["BS"], a["NB"], a["MB"], a["L"], a["scale"],
                                     a["dt"], a["out"], a["ws"], a["wsb"], a["stream"]) == status
    assert words in pk.pa_last_error() and "pa_decode_cached" in pk.pa_last_error()


def call_decode_append(pk, **over):
    a = dict(q=FAKE, nk=FAKE, nv=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE, N=4, H=8, HKV=2, D=128,
             BS=16, NB=100, MB=10, L=160, scale=0.088, dt=2, out=FAKE, ws=FAKE, wsb=0, stream=None)
    a.update(over)
    return pk.lib().pa_decode_append(a["q"], a["nk"], a["nv"], a["k"], a["v"], a["bt"], a["lens"],
                                     a["N"], a["H"], a["HKV"], a["D"], a["BS"], a["NB"], a["MB"],
                                     a["L"], a["scale"], a["dt"], a["out"], a["ws"], a["wsb"],
                                     a["stream"])


@pytest.mark.parametrize("over,status,words", [
    (dict(nk=None), 1, "null"),
    (dict(nv=None), 1, "null"),
    (dict(nv=FAKE + 8), 1, "new_k and new_v must be 16-byte aligned"),
    (dict(D=96), 2, "head_dim"),
    (dict(L=161), 1, "max_seq_len"),
    (dict(L=1000, MB=100, wsb=16), 3, "workspace"),
])
def test_decode_append_rejects_host_visible_errors(pk, over, status, words):
    assert call_decode_append(pk, **over) == status
    assert words in pk.pa_last_error()
    assert "pa_decode_append" in pk.pa_last_error()


def test_decode_append_with_no_sequences_is_a_no_op(pk):
    assert call_decode_append(pk, N=0, q=None, out=None, nk=None, nv=None) == 0


def test_write_and_copy_reject_host_visible_errors(pk):
    L = pk.lib()
    # write: row of 3 f16 elements x 2 heads = 12 bytes is not a multiple of 16
    assert L.pa_write_kv(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 2, 3, 16, 10, 1, None) == 2
    assert "multiple of 16" in pk.pa_last_error()
    assert L.pa_write_kv(FAKE, None, FAKE, FAKE, FAKE, 4, 8, 128, 16, 10, 2, None) == 1
    assert L.pa_write_kv(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 8, 128, 16, 10, 2, None) == 1
    assert L.pa_write_kv(None, None, None, None, None, 0, 8, 128, 16, 10, 2, None) == 0
    assert L.pa_copy_blocks(FAKE, FAKE, None, 3, 16, 8, 128, 10, 2, None) == 1
    assert L.pa_copy_blocks(FAKE, FAKE, FAKE, 3, 16, 8, 128, 10, 9, None) == 1
    assert L.pa_copy_blocks(None, None, None, 0, 16, 8, 128, 10, 2, None) == 0


def test_binding_rejects_cpu_tensors(pk):
    import torch
    q = torch.zeros(1, 4, 64)
    with pytest.raises(ValueError):
        pk.pa_decode(q, torch.zeros(2, 16, 4, 64), torch.zeros(2, 16, 4, 64),
                     torch.zeros(1, 1, dtype=torch.int32), torch.ones(1, dtype=torch.int32), 4,
                     0.125, q, max_seq_len=1)


@pytest.mark.parametrize("N,TQ,H,HKV,D,MQ,L", [(256, 1024, 32, 8, 128, 4, 4096), (16, 8192, 32, 8, 128, 512, 4096),
                                              (1, 4, 64, 8, 128, 4, 32768), (3, 20, 8, 2, 64, 9, 300),
                                              (2, 2, 4, 4, 64, 1, 0)])
def test_multi_query_workspace_formula(pk, N, TQ, H, HKV, D, MQ, L):
    # 64 query rows per workgroup (64 // group query tokens); about 1024 workgroups wanted,
    # partitions of >= 256 tokens, at most 64; with one partition nothing is needed,
    # else (m, l) and head_dim floats per row, head and partition
    g = H // HKV
    # rows per workgroup: 128 when a block has more than 64 rows, else 64 (or 16 for the
    # split variant, which gives one block exactly when 64 rows would)
    tq = (128 if MQ * g > 64 else 64) // g
    items = N * HKV * (-(-MQ // tq))
    parts = max(1, min(-(-1024 // items), -(-L // 256), 64)) if items and L else 1
    up = lambda x: -(-x // 256) * 256
    want = 0 if parts == 1 else up(TQ * H * parts * 2 * 4) + TQ * H * parts * D * 4
    if N > 0:   # a longest-first order of the sequences
        want += up(4 * N)
    rows = MQ * g
    if 1 <= rows <= 16:
        # the rows mode's workspace (the decode kernels' layout with `rows` rows per pair):
        # one wave per 8 tiles of the longest batch (at most 2048), five chunks per wave, a
        # 256-byte header and 16 bytes per chunk, then two partial slots of rows x (D + 2)
        # floats per chunk; the size covers whichever mode the call takes
        waves = min(2048, max(1, -(-(N * HKV * math.ceil(L / 16)) // 8)))
        chunks = 5 * waves
        want = max(want, up(256 + chunks * 16) + up(2 * chunks * rows * 2 * 4) + 2 * chunks * rows * D * 4)
    assert pk.pa_multi_query_workspace_size(N, TQ, H, HKV, D, MQ, L) == want


def call_mq(pk, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE, qs=FAKE, N=1, TQ=4, H=64, HKV=8, D=128,
             BS=16, NB=4000, MB=2048, MQ=4, L=32768, scale=0.088, dt=2, out=FAKE, ws=FAKE, wsb=0,
             stream=None)
    a.update(over)
    return pk.lib().pa_multi_query(a["q"], a["k"], a["v"], a["bt"], a["lens"], a["qs"], a["N"], a["TQ"],
                                   a["H"], a["HKV"], a["D"], a["BS"], a["NB"], a["MB"], a["MQ"], a["L"],
                                   a["scale"], a["dt"], a["out"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("over,status,words", [
    (dict(D=96), 2, "head_dim"),
    (dict(H=9), 1, "multiple"),
    (dict(dt=7), 1, "dtype"),
    (dict(L=32769), 1, "max_seq_len"),
    (dict(MQ=8, L=6, MB=1), 1, "max_q_len"),
    (dict(qs=None), 1, "null"),
    (dict(out=FAKE + 4), 1, "aligned"),
    (dict(scale=float("inf")), 1, "finite"),
    (dict(wsb=16), 3, "workspace"),
    (dict(ws=None, wsb=1 << 30), 3, "workspace"),
    (dict(BS=0), 1, "block_size"),
    (dict(H=65, HKV=1), 2, "at most 64"),
    # a cache slot of 2^24 bytes, or a block of 2^32 bytes (the kernels' 24-bit row and 32-bit
    # block offsets)
    (dict(H=65536, HKV=65536), 2, "per cache slot"),
    (dict(H=8192, HKV=8192, BS=2048, MB=16), 2, "per cache slot"),
])
def test_multi_query_rejects_host_visible_errors(pk, over, status, words):
    assert call_mq(pk, **over) == status
    assert words in pk.pa_last_error()


def test_multi_query_with_no_queries_is_a_no_op(pk):
    assert call_mq(pk, N=0, q=None, out=None) == 0
    assert call_mq(pk, TQ=0, MQ=0, q=None, out=None) == 0


@pytest.mark.parametrize("N,G,H,HKV,D,MG,L", [(256, 32, 40, 40, 128, 8, 1280), (4, 1, 8, 8, 128, 4, 3200),
                                             (8, 2, 32, 8, 128, 6, 150), (3, 3, 16, 1, 64, 1, 40),
                                             (4096, 1024, 8, 8, 128, 32, 32768)])   # tables past 256 MiB
def test_shared_prefix_workspace_formula(pk, N, G, H, HKV, D, MG, L):
    # blocks of 16 / group members per item, about 1024 items wanted, partitions of >= 256
    # tokens, at most 64; a longest-first order of the groups, then (with partitions) the
    # partial results of every sequence, head and partition
    g = H // HKV
    items = G * HKV * (-(-MG // (16 // g)))
    parts = max(1, min(-(-1024 // items), -(-L // 256), 64)) if items and L else 1
    up = lambda x: -(-x // 256) * 256
    want = up(4 * G) + (0 if parts == 1 else up(N * H * parts * 2 * 4) + N * H * parts * D * 4)
    # the rows path (decode kernels): members in blocks of mpb = min(16 / group, MG), each
    # block a laid-out table of at most (mpb + 1) x L tokens rounded to 16-token units and
    # read as 8-token blocks (the largest table); then the block lengths and first rows,
    # after the decode kernels' workspace for mpb x group rows per pair
    mpb = min(16 // g, MG)
    vg = G * (-(-MG // mpb))
    vlen = max(-(-L // 16) * 16 * (mpb + 1), 16)
    if vg <= 2048 and vlen <= 1 << 24 and vg * (vlen // 8) * 4 <= 256 << 20:
        rows = mpb * g
        waves = min(2048, max(1, -(-(N * HKV * math.ceil(L / 16)) // 8)))
        chunks = 5 * waves
        dec = up(256 + chunks * 16) + up(2 * chunks * rows * 2 * 4) + 2 * chunks * rows * D * 4
        total = up(dec) + up(vg * (vlen // 8) * 4) + up(vg * 4) + (vg + 1) * 4
        want = max(want, total)
    assert pk.pa_decode_shared_prefix_workspace_size(N, G, H, HKV, D, MG, L) == want


def call_sp(pk, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE, gs=FAKE, pre=FAKE, N=8, G=2, H=8, HKV=8, D=128,
             BS=16, NB=100, MB=10, MG=4, L=160, scale=0.088, dt=1, out=FAKE, ws=FAKE, wsb=1 << 20,
             stream=None)
    a.update(over)
    return pk.lib().pa_decode_shared_prefix(a["q"], a["k"], a["v"], a["bt"], a["lens"], a["gs"], a["pre"],
                                            a["N"], a["G"], a["H"], a["HKV"], a["D"], a["BS"], a["NB"],
                                            a["MB"], a["MG"], a["L"], a["scale"], a["dt"], a["out"], a["ws"],
                                            a["wsb"], a["stream"])


@pytest.mark.parametrize("over,status,words", [
    (dict(D=96), 2, "head_dim"),
    (dict(dt=0), 2, "float32"),
    (dict(dt=7), 1, "dtype"),
    (dict(H=9), 1, "multiple"),
    (dict(H=34, HKV=2), 2, "at most 16"),
    (dict(L=161), 1, "max_seq_len"),
    (dict(MG=9), 1, "max_group_size"),
    (dict(pre=None), 1, "null"),
    (dict(q=FAKE + 8), 1, "aligned"),
    (dict(scale=float("nan")), 1, "finite"),
    (dict(wsb=0, ws=None), 3, "workspace"),
])
def test_shared_prefix_rejects_host_visible_errors(pk, over, status, words):
    assert call_sp(pk, **over) == status
    assert words in pk.pa_last_error()


def test_shared_prefix_with_no_groups_is_a_no_op(pk):
    assert call_sp(pk, G=0, q=None, out=None) == 0
    assert call_sp(pk, N=0, MG=0, q=None, out=None) == 0
