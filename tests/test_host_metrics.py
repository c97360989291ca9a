"""Host-side measurement logic: the algorithmic byte model every roofline
fraction divides by, and the rocprofv3 summaries (decode durations from a
kernel trace, HBM bytes from counters scaled on a copy, engine clocks) on
synthetic traces (no GPU).

The byte counts are written out here from the cache layouts (codes, scales,
fp16 residual tokens, the fp16 queries read, the fp32 outputs written and
one 4-byte block-table entry per block streamed), independently of
quantized_paged_kv_02_amd.metrics.
"""

import csv
import os

import numpy as np
import pytest

from quantized_paged_kv_02_amd import inputs, metrics, profile_summary

W = inputs.WORKLOADS


def _q_out(batch, hq):
    return batch * hq * 128 * 2 + batch * hq * 128 * 4


@pytest.mark.parametrize("name,layers,want", [
    # INT8, per-token K and V scales: 2 x 128 codes + 2 x 4 B scales per
    # token and KV head (264 B); 4 rows x 2048 tokens x 32 heads; 128 blocks
    ("llama2-7b", 32, 32 * (4 * 2048 * 32 * 264 + 4 * 32 * 128 * 6 + 4 * 128 * 4)),
    # KIVI INT4: nq = 32640 quantized tokens at 128 B codes + 8 B K group
    # scales + 8 B V scales, 128 fp16 window tokens at 512 B; 2040 blocks
    ("kivi-int4", 1, 16 * 8 * (32640 * 144 + 128 * 512) + 16 * 32 * 128 * 6 + 16 * 2040 * 4),
    # Llama-3-70B INT8 per token: 24 rows x 16384 tokens x 8 heads x 264 B
    ("llama3-70b-int8", 80, 80 * (24 * 16384 * 8 * 264 + 24 * 64 * 128 * 6 + 24 * 1024 * 4)),
    # FP8 per tensor: 256 B per token and head, plus the two 4-byte scales
    ("llama3-70b-fp8", 80, 80 * (24 * 16384 * 8 * 256 + 24 * 64 * 128 * 6 + 24 * 1024 * 4 + 8)),
    # unquantized 16-bit caches: 2 x 128 x 2 B per token and head
    ("llama3-70b-fp16", 1, 24 * 16384 * 8 * 512 + 24 * 64 * 128 * 6 + 24 * 1024 * 4),
    ("llama3-70b-bf16", 1, 24 * 16384 * 8 * 512 + 24 * 64 * 128 * 6 + 24 * 1024 * 4),
])
def test_decode_bytes_closed_forms(name, layers, want):
    w = W[name]
    got = metrics.decode_bytes(w.dtype, w.k_gran, w.v_gran, inputs.seq_lens(w), w.num_q_heads,
                               w.num_kv_heads)
    assert got * layers == want


def test_decode_bytes_affine_and_2bit():
    # per quantized token and KV head: affine INT4 adds a 1-byte K zero point
    # per channel and group (2 B per token) and two V zero points (2 B);
    # 2-bit codes take 64 B instead of 128
    for name, per_tok in (("kivi-int4-affine", 148), ("kivi-int2-affine", 84)):
        w = W[name]
        lens = inputs.seq_lens(w)
        got = metrics.decode_bytes(w.dtype, w.k_gran, w.v_gran, lens, w.num_q_heads,
                                   w.num_kv_heads)
        nq, r = 32640, 128
        want = (w.batch * w.num_kv_heads * (nq * per_tok + r * 512)
                + _q_out(w.batch, w.num_q_heads) + w.batch * (nq // 16) * 4)
        assert got == want, name


def test_decode_bytes_ragged_rows_sum_per_row():
    # the ragged GQA workload: the model is a sum over rows
    w = W["llama3-8b-gqa"]
    lens = inputs.seq_lens(w)
    got = metrics.decode_bytes(w.dtype, w.k_gran, w.v_gran, lens, w.num_q_heads, w.num_kv_heads)
    # FP8 per head: 256 B per token and head, 8 per-head scales of K and V
    want = (int(np.sum(lens)) * w.num_kv_heads * 256 + _q_out(w.batch, w.num_q_heads)
            + int(np.sum((lens + 15) // 16)) * 4 + 2 * w.num_kv_heads * 4)
    assert got == want


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        wr.writeheader()
        wr.writerows(rows)


def test_clock_summary(tmp_path):
    """GRBM_GUI_ACTIVE summed over the XCDs / XCD count / duration."""
    d = tmp_path / "run"
    d.mkdir()
    _write_csv(d / "run_agent_info.csv", [
        {"Name": "gfx950", "Num_Xcc": "8", "Max_Engine_Clk_Fcompute": "2400"}])
    # three dispatches: 500 us at 2.2 GHz, then 550 us at 2.0 GHz, and a
    # kernel the pattern does not select
    rows = []
    t = 1_000_000
    for kern, us, ghz in (("kvq_int4_flush_kernel<3>", 500.0, 2.2),
                          ("kvq_int4_flush_kernel<3>", 550.0, 2.0),
                          ("other_kernel", 10.0, 2.0)):
        start, end = t, t + int(us * 1e3)
        rows.append({"Kernel_Name": kern, "Counter_Name": "GRBM_GUI_ACTIVE",
                     "Counter_Value": f"{8 * ghz * (end - start):.1f}",
                     "Start_Timestamp": str(start), "End_Timestamp": str(end)})
        t = end + 100_000
    _write_csv(d / "run_counter_collection.csv", rows)
    out = tmp_path / "clock.md"
    profile_summary.clock(str(tmp_path), "flush", "cmd", str(out))
    text = out.read_text()
    lines = [ln for ln in text.splitlines() if ln.startswith("| 0") or ln.startswith("| 1")]
    assert len(lines) == 2 and "other_kernel" not in text
    cells = [[c.strip() for c in ln.split("|")] for ln in lines]
    assert cells[0][4:6] == ["500.0", "2.200"]
    assert cells[1][3:6] == ["100.0", "550.0", "2.000"]   # 100 us idle before it
    assert "2.40 GHz" in text and "8 XCDs" in text
    assert os.path.exists(out)


def _trace_row(name, start_ns, dur_ns, grid, wg=256):
    return {"Kernel_Name": name, "Start_Timestamp": str(start_ns),
            "End_Timestamp": str(start_ns + dur_ns), "Grid_Size_X": str(grid),
            "Workgroup_Size_X": str(wg)}


def test_decode_times_from_a_trace():
    """Decode dispatches with the launch's own grid, each followed by its
    merge; a decode step's launch with extra flush workgroups (a larger
    grid) and other kernels are left out."""
    rows, t = [], 1_000_000
    for dec_us, red_us in ((100.0, 5.0), (102.0, 4.0), (98.0, 6.0)):
        rows.append(_trace_row("kvq::kvq_paged_decode_int4_kernel<3, true>", t, int(dec_us * 1e3),
                               256 * 256))
        t += int(dec_us * 1e3) + 2_000          # 2 us between decode and merge
        rows.append(_trace_row("kvq::kvq_partition_reduce_kernel", t, int(red_us * 1e3), 16384))
        t += int(red_us * 1e3) + 50_000
    rows.append(_trace_row("kvq::kvq_paged_decode_int4_kernel<3, true>", t, 400_000,
                           300 * 256))                       # flushing step: excluded
    rows.append(_trace_row("at::native::fill", t + 500_000, 3_000, 1024))
    got = profile_summary.decode_times(rows[::-1])           # order by start time
    assert got["dispatches"] == 3 and got["decode_workgroups"] == 256
    assert got["decode_us"] == pytest.approx(100.0)
    assert got["merge_us"] == pytest.approx(5.0)
    assert got["launch_span_us"] == pytest.approx(100.0 + 2.0 + 5.0)
    assert got["decode_median_us"] == pytest.approx(100.0)


def test_traffic_scaled_by_the_copy(tmp_path):
    """Bytes per launch = (median decode + median merge counter, KiB) x
    1024 x (copy size / what the counter reads for the copy)."""
    copy_mib = 1024
    for counter, copy_reads, dec, red in (("FETCH_SIZE", 512 * 1024, [300_000, 310_000, 305_000],
                                           [100, 120]),
                                          ("WRITE_SIZE", 1024 * 1024, [60, 62, 64], [10, 10])):
        d = tmp_path / counter
        d.mkdir()
        rows = [{"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": counter,
                 "Counter_Value": str(v)} for v in (copy_reads, copy_reads, 3.0)]
        rows += [{"Kernel_Name": "kvq_paged_decode_int4_kernel", "Counter_Name": counter,
                  "Counter_Value": str(v)} for v in dec]
        rows += [{"Kernel_Name": "kvq_partition_reduce_kernel", "Counter_Name": counter,
                  "Counter_Value": str(v)} for v in red]
        _write_csv(d / "run_counter_collection.csv", rows)
    out = tmp_path / "traffic.json"
    profile_summary.traffic(str(tmp_path / "FETCH_SIZE"), str(tmp_path / "WRITE_SIZE"),
                            "kivi-int4", copy_mib, "f", "w", str(out), split_tokens=16384)
    import json
    t = json.load(open(out))
    e = t["kivi-int4"]
    assert e["fetch_scale"] == 2.0 and e["write_scale"] == 1.0
    assert e["read_bytes"] == int((305_000 + 110) * 1024 * 2.0)
    assert e["write_bytes"] == int((62 + 10) * 1024 * 1.0)
    assert e["bytes_per_launch"] == e["read_bytes"] + e["write_bytes"]
    assert t["kernel_source_hash"] == profile_summary.kernel_source_hash()
    assert e["dispatches"] == [3, 3] and e["split_tokens"] == 16384


def test_crosscheck_bytes_per_request_from_the_copy(tmp_path):
    """Each request counter becomes bytes with the bytes per request the
    copy shows (copy bytes / its requests): a 64-byte-request counter and a
    128-byte one give the same launch bytes for the same traffic."""
    copy_mib = 256
    copy_bytes = copy_mib << 20
    launch_bytes = 610_000_000          # decode + merge read traffic
    rows = []
    for name, req in (("TCC_EA0_RDREQ_DRAM_sum", 64), ("TCP_TCC_READ_REQ_sum", 128)):
        rows += [{"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": name,
                  "Counter_Value": str(copy_bytes // req)} for _ in range(2)]
        dec = (launch_bytes - 128 * 1024) // req
        rows += [{"Kernel_Name": "kvq_paged_decode_int4_kernel", "Counter_Name": name,
                  "Counter_Value": str(v)} for v in (dec - 10, dec, dec + 10)]
        rows += [{"Kernel_Name": "kvq_partition_reduce_kernel", "Counter_Name": name,
                  "Counter_Value": str(128 * 1024 // req)}]
    _write_csv(tmp_path / "run_counter_collection.csv", rows)
    out = tmp_path / "x.md"
    profile_summary.crosscheck(str(tmp_path), "kivi-int4", copy_mib, "cmd", str(out))
    text = out.read_text()
    for name, req in (("TCC_EA0_RDREQ_DRAM_sum", 64), ("TCP_TCC_READ_REQ_sum", 128)):
        line = next(ln for ln in text.splitlines() if ln.startswith(f"| {name} |"))
        cells = [c.strip() for c in line.split("|")]
        assert cells[3] == f"{req:.2f}"
        assert cells[5] == f"{launch_bytes / 1e6:.2f} MB"
