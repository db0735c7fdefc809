"""GPU parity of pa_multi_query (several causal queries per sequence) against the oracle.

Every batch's query tokens first reach the cache through pa_write_kv, as in a
serving step; the oracle applies the same write and computes each query row's
attention over the sequence's tokens up to its own position, in float64.
Tolerances are those of pa_decode (max-abs 1e-5 fp32, 4e-3 fp16, 8e-3 bf16).
Pools are NaN wherever no token lives, so any read past a row's causal limit,
a sequence end or a table's used entries poisons the output.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import as_numpy
from _gpu import TOL, allowance, assert_close, bits, log, pk, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pk()


def run_gpu(b, d=None, max_q_len=None):
    m = pk()
    d = d or to_dev(b)
    if d.slots is not None:
        m.pa_write_kv(d.new_k, d.new_v, d.slots, d.kc, d.vc)
    qs = b.q_start.cuda()
    out = torch.empty_like(d.q)
    m.pa_multi_query(d.q, d.kc, d.vc, d.bt, d.lens, qs, b.num_kv_heads, b.scale, out,
                     max_q_len=b.max_q_len if max_q_len is None else max_q_len,
                     max_seq_len=b.max_seq_len)
    torch.cuda.synchronize()
    return out, d


def written(b):
    if b.slot_mapping is None:
        return as_numpy(b.k_cache), as_numpy(b.v_cache)
    return oracle.write_kv(as_numpy(b.new_k), as_numpy(b.new_v), as_numpy(b.slot_mapping),
                           as_numpy(b.k_cache), as_numpy(b.v_cache))


def run_oracle(b):
    kc, vc = written(b)
    return oracle.paged_multi_query(as_numpy(b.q), kc, vc, as_numpy(b.block_tables),
                                    as_numpy(b.seq_lens), as_numpy(b.q_start), b.scale, b.dtype)


def batch(seed, dtype, lens, queries, Hq, Hkv, D, B, extra=4):
    g = torch.Generator().manual_seed(seed)
    return workloads._paged(name=f"mq{seed}", dtype=dtype, lens=lens, Hq=Hq, Hkv=Hkv, D=D, B=B,
                            num_blocks=sum(-(-L // B) for L in lens) + extra, gen=g, queries=queries)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_small_batch(dtype):
    b = workloads.multi_query_small(dtype=dtype)
    log(f"multi_query_small {dtype}")
    out, _ = run_gpu(b)
    assert_close(out.float().cpu().double().numpy(), run_oracle(b), dtype, "small")


SWEEP = [  # dtype, D, B, Hq, Hkv, lens, queries
    ("bf16", 128, 16, 32, 8, [1, 40, 97, 300, 64], [1, 40, 5, 130, 64]),
    ("f16", 128, 8, 8, 8, [33, 100, 17], [33, 7, 16]),
    ("bf16", 64, 32, 16, 1, [250, 3, 64], [70, 3, 1]),
    ("f16", 64, 16, 12, 3, [129, 31], [65, 31]),
    ("bf16", 128, 5, 64, 8, [77, 200], [9, 8]),
    ("f32", 128, 16, 8, 2, [45, 90], [20, 90]),
    ("bf16", 128, 16, 40, 40, [18, 260], [18, 33]),
    # at most 16 rows per (sequence, KV head), block sizes 8/16/32: the decode kernels'
    # rows mode (each pair's rows in the 16 columns of a score tile)
    ("f16", 64, 16, 16, 8, [5, 300, 33], [5, 8, 1]),
    ("bf16", 128, 8, 16, 1, [40, 1, 77], [1, 1, 1]),
    ("bf16", 64, 32, 4, 4, [700, 16, 90], [16, 16, 2]),
    ("bf16", 128, 16, 32, 8, [31, 64, 65, 200], [4, 4, 3, 4]),
    ("bf16", 128, 16, 32, 8, [1, 2, 3, 17, 33, 300], [0, 2, 1, 2, 0, 2]),    # 8 rows, no-query sequences
    ("f16", 128, 8, 12, 4, [5000, 3, 4099], [4, 3, 1]),                      # split pairs, 12 rows
    # the same row counts with other block sizes: the split variant (four waves split the context)
    ("bf16", 128, 5, 32, 8, [31, 64, 65, 200], [4, 4, 3, 4]),
    ("f16", 64, 12, 16, 8, [5, 300, 33], [5, 8, 1]),
]


@pytest.mark.parametrize("case", range(len(SWEEP)))
def test_shape_sweep(case):
    dt, D, B, Hq, Hkv, lens, qn = SWEEP[case]
    b = batch(100 + case, dt, lens, qn, Hq, Hkv, D, B)
    log(f"sweep {SWEEP[case]}")
    out, _ = run_gpu(b)
    assert_close(out.float().cpu().double().numpy(), run_oracle(b), dt, f"sweep {case}")


def _random_shared_tile_case(seed):
    # a seeded draw of shapes that take the shared-tile (pipelined for 16-bit types) path:
    # more than 16 rows per (sequence, KV head) in the longest sequence
    r = np.random.default_rng(seed)
    dt = ["bf16", "f16", "bf16", "f16", "f32"][seed % 5]
    D = int(r.choice([64, 128]))
    g = int(r.choice([1, 2, 4, 8]))
    Hkv = int(r.choice([1, 2, 4]))
    B = int(r.choice([4, 5, 8, 11, 16, 32]))
    n = int(r.integers(1, 5))
    queries = [int(r.integers(0, 90)) for _ in range(n)]
    queries[int(r.integers(0, n))] = int(r.integers(max(17, 17 // g + 1), 150))   # one long chunk
    lens = [q + int(r.integers(0, 400)) for q in queries]
    return dt, D, B, g * Hkv, Hkv, lens, queries


@pytest.mark.parametrize("seed", range(12))
def test_random_shared_tile_shapes(seed):
    dt, D, B, Hq, Hkv, lens, qn = _random_shared_tile_case(seed)
    b = batch(300 + seed, dt, lens, qn, Hq, Hkv, D, B)
    log(f"random shared-tile case {seed}: {dt} D={D} B={B} Hq={Hq} Hkv={Hkv} lens={lens} queries={qn}")
    out, _ = run_gpu(b)
    assert_close(out.float().cpu().double().numpy(), run_oracle(b), dt, f"random case {seed}")


@pytest.mark.parametrize("dtype,scale,queries", [
    ("bf16", -0.09, [4, 2, 1]),     # at most 16 rows per (sequence, KV head): split variant
    ("bf16", -0.09, [40, 70, 1]),   # shared-tile variant
    ("f16", 0.0, [4, 2, 1]),
    ("f16", 0.0, [40, 70, 1]),
    ("f32", -0.2, [40, 70, 1]),
    ("bf16", 0.0, [40, 70, 1]),
])
def test_negative_and_zero_scale(dtype, scale, queries):
    # a negative scale reverses the ordering of the scores (the kernel flips the sign of
    # q and uses the magnitude); scale 0 gives every visible token the same weight
    b = batch(31, dtype, [90, 200, 33], queries, 16, 4, 128, 16)
    b.scale = scale
    log(f"scale {scale} {dtype} queries {queries}")
    out, _ = run_gpu(b)
    assert_close(out.float().cpu().double().numpy(), run_oracle(b), dtype, f"scale {scale}")


def test_long_context_few_queries_uses_partitions():
    # one sequence, 3 queries, 5000 tokens: the rows mode cuts its pairs over many waves
    # and the merge kernel folds the pieces
    b = batch(7, "bf16", [5000], [3], 8, 8, 128, 16)
    m = pk()
    assert m.pa_multi_query_workspace_size(1, 3, 8, 8, 128, 3, 5000) > 0
    log("partitioned long context")
    out, _ = run_gpu(b)
    assert_close(out.float().cpu().double().numpy(), run_oracle(b), "bf16", "partitions")


@pytest.mark.parametrize("dtype,B,scale", [("bf16", 16, None), ("f16", 7, None), ("bf16", 16, 0.0)])
def test_long_context_many_queries_partitions_on_shared_tiles(dtype, B, scale):
    # one sequence of 5000 tokens whose last 40 are queries, 4 heads per KV head: 160 rows per
    # KV head, so the shared-tile loop runs (two 128-row blocks), and with 4 items the context
    # of each is cut into partitions; the masked last tiles fall inside the last partition
    b = batch(8, dtype, [5000], [40], 8, 2, 128, B)
    if scale is not None:
        b.scale = scale
    m = pk()
    assert m.pa_multi_query_workspace_size(1, 40, 8, 2, 128, 40, 5000) > 0
    log(f"partitioned shared tiles {dtype} B={B} scale={b.scale}")
    out, _ = run_gpu(b)
    assert_close(out.float().cpu().double().numpy(), run_oracle(b), dtype, "partitions, shared tiles")


def test_one_query_per_sequence_matches_decode():
    b = batch(9, "bf16", [1, 17, 300, 1000, 64, 2], [1] * 6, 32, 8, 128, 16)
    m = pk()
    log("one query per sequence vs pa_decode")
    out, d = run_gpu(b)
    dec = torch.empty_like(d.q)
    m.pa_decode(d.q, d.kc, d.vc, d.bt, d.lens, b.num_kv_heads, b.scale, dec, max_seq_len=b.max_seq_len)
    torch.cuda.synchronize()
    ref = run_oracle(b)
    assert_close(out.float().cpu().double().numpy(), ref, "bf16", "mq")
    assert_close(dec.float().cpu().double().numpy(), ref, "bf16", "decode")


def test_max_q_len_larger_than_needed_and_deterministic():
    b = batch(11, "f16", [50, 120, 7], [10, 120, 7], 16, 4, 128, 16)
    log("max_q_len slack, determinism")
    out1, d = run_gpu(b, max_q_len=120)
    out2, _ = run_gpu(b, d=d, max_q_len=120)
    assert torch.equal(bits(out1.cpu()), bits(out2.cpu()))
    assert_close(out1.float().cpu().double().numpy(), run_oracle(b), "f16", "slack")


def test_many_short_sequences_in_longest_first_order():
    # more sequences than the ordering pass has threads, lengths 1..80, 1..4 queries each
    rng = np.random.default_rng(21)
    lens = rng.integers(1, 81, 1500).tolist()
    qn = [int(min(L, q)) for L, q in zip(lens, rng.integers(1, 5, 1500))]
    b = batch(21, "bf16", lens, qn, 32, 8, 128, 16)
    log("1500 short sequences")
    out, _ = run_gpu(b)
    assert_close(out.float().cpu().double().numpy(), run_oracle(b), "bf16", "many")


def test_more_sequences_than_the_ordering_pass_sorts_in_one_sweep():
    # 2100 short sequences (more than twice the ordering pass's 1024 threads, and more
    # than the decode kernels keep in LDS, so the split variant runs), up to 16 (query,
    # head) rows per KV head; some have no queries
    rng = np.random.default_rng(23)
    lens = rng.integers(1, 61, 2100).tolist()
    qn = [int(min(L, q)) for L, q in zip(lens, rng.integers(0, 5, 2100))]
    b = batch(23, "f16", lens, qn, 16, 4, 64, 8)
    log("2100 sequences")
    out, _ = run_gpu(b)
    assert_close(out.float().cpu().double().numpy(), run_oracle(b), "f16", "2100")


@pytest.mark.parametrize("name,make", [
    ("spec", lambda: workloads.llama3_8b_spec(num_seqs=12, num_blocks=5000)),
    ("chunk", lambda: workloads.llama3_8b_chunk(num_seqs=2, chunk=96, max_prior=500)),
])
def test_workloads_reduced(name, make):
    b = make()
    log(f"{name} reduced")
    out, _ = run_gpu(b)
    assert_close(out.float().cpu().double().numpy(), run_oracle(b), "bf16", name)


@pytest.mark.parametrize("exp2", [16, 20, 100])
def test_bf16_values_far_outside_the_unit_range(exp2):
    # bf16 prefill-sized blocks stage V in LDS as fp16, which holds |v| < 2^16 exactly; a
    # larger value turns the workgroup's result non-finite and the workgroup runs again with
    # bf16 V.  One V row (every KV head) of two sequences is multiplied by 2^exp2 (exact in
    # bf16) and every query of those sequences attends to it (it is in the prompt), so the
    # outputs range from O(1) to about 2^exp2.  All must be finite, and within the usual
    # bound plus 2^-9 of the largest |V| the sequence holds: bf16 precision at the scale of
    # the values being averaged.
    b = batch(41 + exp2, "bf16", [300, 90, 700], [40, 64, 33], 32, 8, 128, 16)
    vflat = b.v_cache.view(-1, 8, 128)
    for s, t in ((0, 5), (2, 70)):
        slot = int(b.block_tables[s, t // 16]) * 16 + t % 16
        vflat[slot] = (vflat[slot].float() * 2.0 ** exp2).to(torch.bfloat16)
    log(f"bf16 V rows x 2^{exp2}")
    out, _ = run_gpu(b)
    got = out.float().cpu().double().numpy()
    assert np.isfinite(got).all()
    ref = run_oracle(b)
    qs = b.q_start.tolist()
    _, vc = written(b)
    vmax = np.zeros(b.q.shape[0])
    for s in range(b.num_seqs):
        V = oracle.to_f64(oracle.gather(vc, as_numpy(b.block_tables)[s], int(b.seq_lens[s]), b.block_size),
                          "bf16")
        vmax[qs[s]:qs[s + 1]] = np.abs(V).max()
    bound = allowance(ref, "bf16") + 2.0 ** -9 * vmax[:, None, None]
    err = np.abs(got - ref)
    assert (err <= bound).all(), f"{(err > bound).sum()} outputs over the bound, max err {err.max():.3e}"
    log(f"V x 2^{exp2}: max err {err.max():.3e}, max |out| {np.abs(ref).max():.3e}")


def oracle_rows(b, rows):
    """Oracle output for the given query rows (full-size batches): each sequence's K/V is
    gathered once, and each row attends to its causal prefix of it."""
    kc, vc = written(b)
    qs = b.q_start.tolist()
    lens = b.seq_lens.tolist()
    bt = as_numpy(b.block_tables)
    by_seq = {}
    for r in rows:
        by_seq.setdefault(int(np.searchsorted(qs, r, side="right") - 1), []).append(r)
    res = {}
    for s, rs in by_seq.items():
        n, L = qs[s + 1] - qs[s], lens[s]
        last = max(L - n + (r - qs[s]) for r in rs)
        K = oracle.to_f64(oracle.gather(kc, bt[s], last + 1, b.block_size), b.dtype)
        V = oracle.to_f64(oracle.gather(vc, bt[s], last + 1, b.block_size), b.dtype)
        for r in rs:
            pos = L - n + (r - qs[s])
            res[r] = oracle.attend(oracle.to_f64(as_numpy(b.q[r]), b.dtype), K[:pos + 1], V[:pos + 1],
                                   b.scale)
    return np.stack([res[r] for r in rows])


def test_full_size_speculative_verification_every_row():
    b = workloads.WORKLOADS["llama3_8b_spec"]()
    log("llama3_8b_spec full size")
    out, _ = run_gpu(b)
    got = out.float().cpu().double().numpy()
    assert np.isfinite(got).all()
    rows = list(range(b.q.shape[0]))
    err = assert_close(got, oracle_rows(b, rows), "bf16", "llama3_8b_spec")
    log(f"llama3_8b_spec: all {len(rows)} query rows x {b.num_heads} heads compared, max abs err {err:.3e}")


def test_full_size_chunked_prefill_every_query_block():
    # one row from every 16-query block of every sequence (a different offset in each
    # block), plus each sequence's first and last query
    b = workloads.WORKLOADS["llama3_8b_chunk"]()
    log("llama3_8b_chunk full size")
    out, _ = run_gpu(b)
    got = out.float().cpu().double().numpy()
    assert np.isfinite(got).all()
    rng = np.random.default_rng(0)
    qs = b.q_start.tolist()
    rows = set()
    for s in range(b.num_seqs):
        rows |= {qs[s], qs[s + 1] - 1}
        for a in range(qs[s], qs[s + 1], 16):
            rows.add(int(a + rng.integers(0, min(16, qs[s + 1] - a))))
    rows = sorted(rows)
    err = assert_close(got[rows], oracle_rows(b, rows), "bf16", "llama3_8b_chunk")
    log(f"llama3_8b_chunk: {len(rows)} of {b.q.shape[0]} query rows x {b.num_heads} heads compared "
        f"(every 16-query block of all {b.num_seqs} sequences), max abs err {err:.3e}")
