"""Host logic of bench.py, on the CPU: the HBM traffic it derives from rocprofv3 counter
files, the distinct bytes of a batch whose sequences share blocks, the test that lets a step
run as one pa_decode_append call, and the refusal of more than one GPU."""

import csv
import json
import os
import subprocess
import sys

import pytest

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def write_counters(path, counter, rows):
    """A counter_collection file as rocprofv3 --pmc -f csv writes it: one row per dispatch,
    counter and hardware instance group (rows of one dispatch are summed)."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for disp, kernel, value in rows:
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": kernel, "Counter_Name": counter,
                        "Counter_Value": value})


DEC = "void pagedkv::decode_kernel<2, 128, 16, 4, true, true, false>(pagedkv::DecodeParams)"
RED = "void pagedkv::reduce_kernel<2, 128, 4, false>(pagedkv::DecodeParams)"
TORCH_RED = "void at::native::reduce_kernel<512, 1>(...)"   # the cache flush's sum
COPY = "pagedkv::copy_blocks_kernel(...)"


def test_record_traffic_scales_each_counter_by_the_copy_calibration(tmp_path, monkeypatch):
    # the calibration copy moves 1 GiB each way: FETCH_SIZE reads half of it (scale 2),
    # WRITE_SIZE all of it (scale 1)
    cal_f, cal_w = tmp_path / "cf.csv", tmp_path / "cw.csv"
    write_counters(cal_f, "FETCH_SIZE", [(1, COPY, 524288.0), (2, COPY, 524288.0)])
    write_counters(cal_w, "WRITE_SIZE", [(1, COPY, 1048576.0)])
    dec_f, dec_w = tmp_path / "df.csv", tmp_path / "dw.csv"
    # dispatch 10 is reported in two rows (two instance groups): 600 + 400 KiB
    write_counters(dec_f, "FETCH_SIZE", [(10, DEC, 600.0), (10, DEC, 400.0), (12, DEC, 1200.0),
                                         (11, RED, 10.0), (13, RED, 30.0), (14, TORCH_RED, 9e9)])
    write_counters(dec_w, "WRITE_SIZE", [(10, DEC, 50.0), (12, DEC, 70.0), (11, RED, 5.0),
                                         (13, RED, 5.0), (14, TORCH_RED, 9e9)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    bench.record_traffic([str(dec_f), str(dec_w), str(cal_f), str(cal_w)])
    t = json.loads(out.read_text())
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    dec, red = t["per_kernel"]["pagedkv::decode_kernel"], t["per_kernel"]["pagedkv::reduce_kernel"]
    assert dec["fetch_kib"] == pytest.approx(1100.0) and dec["dispatches"] == [2, 2]
    assert red["fetch_kib"] == pytest.approx(20.0) and red["write_kib"] == pytest.approx(5.0)
    want = (1100 * 2 + 60) * 1024 + (20 * 2 + 5) * 1024   # the flush's reduction is not counted
    assert t["hbm_bytes_per_call"] == pytest.approx(want)
    # the bench line reports it only for the kernel sources it was taken on
    assert t["kernel_sha"] == bench.kernel_sha()
    assert bench.measured_traffic() == pytest.approx(want)
    t["kernel_sha"] = "0" * 16
    out.write_text(json.dumps(t))
    assert bench.measured_traffic() is None


def test_distinct_bytes_count_each_shared_slot_once():
    b = workloads.opt13b_shared(num_prompts=2, samples=3, prompt_len=48, tail_max=20)
    B = b.block_size
    slots = set()
    for s, L in enumerate(b.seq_lens.tolist()):
        for t in range(L):
            slots.add((int(b.block_tables[s, t // B]), t % B))
    row = b.num_kv_heads * b.head_dim * 2 * 2      # K and V, fp16
    assert bench.unique_kv_bytes(b) == len(slots) * row
    # the samples do share their prompt: fewer distinct slots than tokens
    assert len(slots) < int(b.seq_lens.sum())


def test_one_call_step_needs_each_sequences_newest_slot():
    b = workloads.llama3_8b(num_seqs=6, min_len=5, max_len=40, num_blocks=32)
    assert bench.write_is_newest(b)
    b.slot_mapping = b.slot_mapping.clone()
    b.slot_mapping[2] += 1 if int(b.slot_mapping[2]) % b.block_size else -1  # another slot of the pool
    assert not bench.write_is_newest(b)
    b.slot_mapping = None
    assert not bench.write_is_newest(b)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
