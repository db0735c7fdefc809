"""GPU parity of pa_decode_shared_prefix: pa_decode's result, each group's shared
prefix read once.

The expected output is the decode oracle itself (softmax over every token of
each sequence): sharing changes only how often blocks are read.  Groups are
built with the reference block manager -- a prompt allocated once, forked into
the group's members, each member then appending its own tail (copy-on-write of a
shared, partly filled last block included) -- so the tables really share their
leading blocks.  Pools are NaN wherever no token lives.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import TORCH_DTYPE, as_numpy
from _gpu import assert_close, bits, log, pk, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pk()


def grouped_batch(seed, dtype, groups, Hq, Hkv, D, B):
    """groups: list of (prompt_len, [tail lengths of the members])."""
    rng = np.random.default_rng(seed)
    g = torch.Generator().manual_seed(seed)
    need = sum(-(-P // B) + sum(-(-t // B) + 1 for t in tails) for P, tails in groups) + 4
    bm = oracle.BlockManager(need, B, free_order=rng.permutation(need))
    tdt = TORCH_DTYPE[dtype]
    kc = torch.full((need, B, Hkv, D), float("nan"), dtype=tdt)
    vc = torch.full_like(kc, float("nan"))
    kf, vf = kc.view(-1, Hkv, D), vc.view(-1, Hkv, D)
    seqs, prefix = [], []
    sid = 0
    for P, tails in groups:
        lead = sid
        bm.allocate(lead, P)
        rows = (torch.randn(P, 2, Hkv, D, generator=g) * 0.7).to(tdt)
        for t in range(P):
            slot = bm.slot(lead, t)
            kf[slot], vf[slot] = rows[t, 0], rows[t, 1]
        members = [lead] + [lead + i for i in range(1, len(tails))]
        for m_ in members[1:]:
            bm.fork(lead, m_)
        for m_, tail in zip(members, tails):
            for _ in range(tail):
                slot, cow = bm.append_slot(m_)
                if cow:
                    src, dst = cow
                    kc[dst], vc[dst] = kc[src].clone(), vc[src].clone()
                r = (torch.randn(2, Hkv, D, generator=g) * 0.7).to(tdt)
                kf[slot], vf[slot] = r[0], r[1]
        # shared prefix: the leading table entries every member still has in common
        tabs = [bm.tables[m_] for m_ in members]
        nb = -(-P // B)
        same = 0
        while same < nb and all(t[same] == tabs[0][same] for t in tabs):
            same += 1
        prefix.append(P if same == nb else same * B)
        seqs += members
        sid += len(tails)
    N = len(seqs)
    lens = [bm.lens[s] for s in seqs]
    mb = max(1, max(len(bm.tables[s]) for s in seqs))
    bt = torch.full((N, mb), -1, dtype=torch.int32)
    for i, s in enumerate(seqs):
        bt[i, :len(bm.tables[s])] = torch.tensor(bm.tables[s], dtype=torch.int32)
    q = (torch.randn(N, Hq, D, generator=g)).to(tdt)
    b = workloads.PagedBatch(name=f"groups{seed}", dtype=dtype, num_heads=Hq, num_kv_heads=Hkv,
                             head_dim=D, block_size=B, num_blocks=need, scale=D ** -0.5, q=q,
                             k_cache=kc, v_cache=vc, block_tables=bt,
                             seq_lens=torch.tensor(lens, dtype=torch.int32),
                             seq_lens_before=torch.tensor(lens, dtype=torch.int32))
    sizes = [len(t) for _, t in groups]
    b.group_start = torch.tensor(np.concatenate([[0], np.cumsum(sizes)]), dtype=torch.int32)
    b.prefix_lens = torch.tensor(prefix, dtype=torch.int32)
    return b


def run(b, d=None, max_group_size=None):
    m = pk()
    d = d or to_dev(b)
    out = torch.empty_like(d.q)
    mg = int((b.group_start[1:] - b.group_start[:-1]).max()) if max_group_size is None else max_group_size
    m.pa_decode_shared_prefix(d.q, d.kc, d.vc, d.bt, d.lens, b.group_start.cuda(), b.prefix_lens.cuda(),
                              b.num_kv_heads, b.scale, out, max_group_size=mg,
                              max_seq_len=b.max_seq_len)
    torch.cuda.synchronize()
    return out, d


def oracle_out(b, seqs=None):
    return oracle.paged_decode(as_numpy(b.q), as_numpy(b.k_cache), as_numpy(b.v_cache),
                               as_numpy(b.block_tables), as_numpy(b.seq_lens), b.scale, b.dtype, seqs=seqs)


CASES = [  # dtype, Hq, Hkv, D, B, groups
    ("f16", 8, 8, 128, 16, [(64, [0, 5, 17, 40]), (33, [1, 0, 2]), (16, [7])]),
    ("bf16", 32, 8, 128, 16, [(100, [3, 9, 0, 31, 50, 2]), (48, [16, 16])]),   # 6 members, g=4: 2 blocks
    ("bf16", 16, 1, 64, 8, [(20, [1]), (9, [0])]),                             # g=16: one member per block
    ("f16", 12, 3, 64, 32, [(0, [5, 9, 40]), (70, [0, 0, 0])]),                # empty prefix; no tails
    ("bf16", 64, 8, 128, 5, [(61, [4, 4, 12])]),                               # odd block size, g=8
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_groups_match_the_decode_oracle(case):
    dt, Hq, Hkv, D, B, groups = CASES[case]
    b = grouped_batch(40 + case, dt, groups, Hq, Hkv, D, B)
    log(f"shared prefix case {case}: {CASES[case]}, prefixes {b.prefix_lens.tolist()}")
    out, _ = run(b)
    assert_close(out.float().cpu().double().numpy(), oracle_out(b), dt, f"case {case}")


@pytest.mark.parametrize("case", range(len(CASES)))
def test_split_kernel_matches_the_decode_oracle(case, monkeypatch):
    # the same groups on the split multi-query kernel (the path for block sizes outside
    # {8, 16, 32}, batches beyond the decode kernels' tables and ids of 2^22 blocks or more)
    monkeypatch.setenv("PA_SHARED_PREFIX_ROWS", "0")
    dt, Hq, Hkv, D, B, groups = CASES[case]
    b = grouped_batch(40 + case, dt, groups, Hq, Hkv, D, B)
    log(f"shared prefix case {case} on the split kernel")
    out, _ = run(b)
    assert_close(out.float().cpu().double().numpy(), oracle_out(b), dt, f"split, case {case}")


# Groups for the decode kernels' rows path: each block of members gets a laid-out table
# (the prefix rounded down to whole 16-token units, or 32-token blocks, then every member's
# own tokens padded to whole units), member i of a block is row i.
ROWS_CASES = [  # dtype, Hq, Hkv, D, B, groups
    ("f16", 8, 8, 128, 16, [(0, [0, 5, 0, 16, 1]), (0, [0])]),   # empty members: zeros
    ("bf16", 8, 8, 64, 16, [(40, list(range(20)))]),             # 20 members, g=1: rows 0..15, then 4
    ("bf16", 32, 8, 128, 32, [(64, [5, 40, 17]), (96, [0, 33])]),  # 32-token blocks: half-block tiles
    ("f16", 16, 4, 128, 8, [(24, [3, 8, 9, 0]), (8, [1, 15])]),  # prefix 24 in 8-token blocks: 16 shared
    ("bf16", 64, 8, 128, 16, [(100, [1, 2]), (17, [30]), (250, [0, 0])]),  # g=8: 2 members per block
]


@pytest.mark.parametrize("case", range(len(ROWS_CASES)))
def test_rows_path_groups(case):
    dt, Hq, Hkv, D, B, groups = ROWS_CASES[case]
    b = grouped_batch(70 + case, dt, groups, Hq, Hkv, D, B)
    log(f"shared prefix rows case {case}: {ROWS_CASES[case]}, prefixes {b.prefix_lens.tolist()}")
    out, d = run(b)
    got = out.float().cpu().double().numpy()
    assert_close(got, oracle_out(b), dt, f"rows case {case}")
    empty = (b.seq_lens == 0).numpy()
    assert (got[empty] == 0).all(), "empty members must get zeros"
    out2, _ = run(b, d=d)
    assert torch.equal(bits(out.cpu()), bits(out2.cpu())), "reruns differ"


def test_rows_path_long_prefix_split_over_waves():
    # 2 groups x 8 KV heads, each pair thousands of tokens: pairs are cut over many waves
    # and merged; members' own tokens sit after the prefix in the laid-out table
    b = grouped_batch(81, "bf16", [(4000, [1, 300, 0, 77, 16, 5]), (2500, [640, 2])], 32, 8, 128, 16)
    log("shared prefix rows: long prefixes")
    out, _ = run(b)
    assert_close(out.float().cpu().double().numpy(), oracle_out(b), "bf16", "long prefixes")


@pytest.mark.parametrize("scale", [-0.11, 0.0])
def test_negative_and_zero_scale(scale):
    b = grouped_batch(61, "bf16", [(64, [0, 5, 17, 40]), (33, [1, 0, 2])], 32, 8, 128, 16)
    b.scale = scale
    log(f"shared prefix, scale {scale}")
    out, _ = run(b)
    assert_close(out.float().cpu().double().numpy(), oracle_out(b), "bf16", f"scale {scale}")


def test_many_groups_in_longest_first_order():
    # more groups than the ordering pass has threads
    rng = np.random.default_rng(3)
    groups = [(int(rng.integers(1, 40)), [int(x) for x in rng.integers(0, 20, int(rng.integers(1, 4)))])
              for _ in range(1100)]
    b = grouped_batch(3, "f16", groups, 8, 8, 64, 8)
    log("1100 groups")
    out, _ = run(b)
    assert_close(out.float().cpu().double().numpy(), oracle_out(b), "f16", "many groups")


def test_long_prefix_few_groups_uses_partitions_and_matches_pa_decode():
    b = grouped_batch(7, "f16", [(3000, [10, 200, 0, 77])], 8, 8, 128, 16)
    m = pk()
    assert m.pa_decode_shared_prefix_workspace_size(4, 1, 8, 8, 128, 4, b.max_seq_len) > 0
    log("shared prefix: partitions")
    out, d = run(b)
    dec = torch.empty_like(d.q)
    m.pa_decode(d.q, d.kc, d.vc, d.bt, d.lens, b.num_kv_heads, b.scale, dec, max_seq_len=b.max_seq_len)
    torch.cuda.synchronize()
    ref = oracle_out(b)
    assert_close(out.float().cpu().double().numpy(), ref, "f16", "shared")
    assert_close(dec.float().cpu().double().numpy(), ref, "f16", "decode")
    out2, _ = run(b, d=d)
    assert torch.equal(bits(out.cpu()), bits(out2.cpu()))


@pytest.mark.parametrize("name,make", [
    ("opt13b_shared", lambda: workloads.opt13b_shared(num_prompts=3, samples=8, prompt_len=256, tail_max=64)),
    ("opt13b_cow", lambda: workloads.opt13b_cow(num_prompts=2, samples=8, prompt_len=250)),
])
def test_workloads_reduced(name, make):
    b = make()
    m = pk()
    d = to_dev(b)
    if b.cow_pairs is not None:
        m.pa_copy_blocks(d.kc, d.vc, d.pairs)
        m.pa_write_kv(d.new_k, d.new_v, d.slots, d.kc, d.vc)
        kc, vc = oracle.copy_blocks(as_numpy(b.k_cache), as_numpy(b.v_cache), as_numpy(b.cow_pairs))
        kc, vc = oracle.write_kv(as_numpy(b.new_k), as_numpy(b.new_v), as_numpy(b.slot_mapping), kc, vc)
    else:
        kc, vc = as_numpy(b.k_cache), as_numpy(b.v_cache)
    log(f"{name} reduced")
    out, _ = run(b, d=d)
    ref = oracle.paged_decode(as_numpy(b.q), kc, vc, as_numpy(b.block_tables), as_numpy(b.seq_lens),
                              b.scale, "f16")
    assert_close(out.float().cpu().double().numpy(), ref, "f16", name)


def test_full_size_opt13b_shared_every_sequence():
    b = workloads.opt13b_shared()
    log("opt13b_shared full size")
    out, _ = run(b)
    got = out.float().cpu().double().numpy()
    assert np.isfinite(got).all()
    err = assert_close(got, oracle_out(b), "f16", "opt13b_shared")
    log(f"opt13b_shared: all {b.num_seqs} sequences x {b.num_heads} heads compared, max abs err {err:.3e}")
