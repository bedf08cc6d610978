"""Host logic of bench.py on the CPU: the algorithmic byte model against the
closed-form totals of the method (every mandated buffer written once and read
once by the next stage), the partial-row count against brute force, the
counter scaling and trace tables on small synthetic profiler databases, the
source hash's indifference to comments, and the one-GPU guard."""
import json
import os
import sqlite3
import subprocess
import sys

import pytest

import bench
from workloads import CONFIGS, make_routing

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _closed_form(cfg, transport="staged"):
    """Row-payload bytes of one dispatch+combine: x read once per token; each
    dispatch row written by pack, read+written by the transfer, read+written by
    the shuffle (5 row passes; 3 when pack writes the receive rows itself);
    each expert output row read by combine-send and written to the return
    buffer, read+written by the transfer back, read by the reduce (5 passes;
    3 when combine-send writes the return rows itself); one x-sized output."""
    N, T, K, H = cfg.N, cfg.T, cfg.K, cfg.H
    R = N * T * K
    hb = (H + 4 * (H // 128)) if cfg.dtype == "fp8" else 2 * H
    passes_d, passes_c = (5, 5) if transport == "staged" else (3, 3)
    return N * T * H * 2 + passes_d * R * hb + passes_c * R * 2 * H + N * T * H * 2


@pytest.mark.parametrize("key", ["A", "B", "C", "D", "E"])
@pytest.mark.parametrize("transport", ["staged", "direct"])
def test_byte_model_matches_closed_form(key, transport):
    cfg = CONFIGS[key]
    kb = bench.kernel_bytes(cfg, transport)
    total = sum(kb.values())
    main = _closed_form(cfg, transport)
    # the rest is metadata: a few int32 per row (ids, positions, meta words,
    # the receiver's 20 bytes of row maps) and the per-rank tables
    R, N, E = cfg.rows, cfg.N, cfg.E
    small = 96 * R + 64 * N * E + 16 * N * (N + 1) + 64 * E
    assert main <= total <= main + small, (total, main)


def test_headline_totals():
    """The DeepSeek-R1 decode totals: 4.817 GB staged (602 us at 8 TB/s),
    2.938 GB with direct push (367 us); of them 726 408 bytes are the
    receiver's map kernel: forming the group offsets (32 x 256 counts and
    32 x 257 send offsets in; 32 x 33 receive offsets, 33 receive bases and
    257 expert offsets out, 4 bytes each) and writing 20 bytes of maps per
    row.  The route plan (no group offsets here: the pack runs in send-row
    order) reads idx and writes counts, send offsets (row- and column-major),
    positions and each send row's item."""
    c = CONFIGS["C"]
    maps = 4 * (32 * 256 + 32 * 257 + 32 * 33 + 33 + 257) + 32768 * 20
    kb = bench.kernel_bytes(c)
    assert kb["recv_map"] == maps == 726_408
    assert kb["route_plan"] == 4 * (3 * 32768 + 32 * 256 + 2 * 32 * 257)
    assert sum(kb.values()) == 4_817_459_852
    assert sum(bench.kernel_bytes(c, "direct").values()) == 2_938_149_516
    # fixed slots: 4 more bytes of maps per row (the slot of each receive row)
    fx = bench.kernel_bytes(c, layout="fixed")
    assert sum(fx.values()) == sum(kb.values()) + 32768 * 4
    # the packed layout's token-order pack (a sender's tokens above 2 MiB)
    # needs the group offsets from the route plan too
    big = c.with_(T=256)
    assert bench.kernel_bytes(big)["route_plan"] > bench.kernel_bytes(big, layout="fixed")["route_plan"]


def test_byte_model_follows_the_librarys_rules():
    """The byte model's pack-order boundary and record-sum limit are the
    library's (read from the kernel interface header), and the group offsets
    are counted in the route plan exactly where the library forms them there:
    the token-order pack (unless its rows go to fixed slots with the
    receiver-side combine), and the partial combine's records in the
    send-row-order pack past the record-sum limit."""
    import re
    hdr = open(os.path.join(ROOT, "combine_moe_dispatch_amd", "csrc", "moe_kernels.h")).read()
    m = re.search(r"PACK_ROWS_MAX_SENDER_BYTES\s*=\s*(\d+)\s*<<\s*(\d+)", hdr)
    assert m and bench.PACK_ROWS_MAX_SENDER_BYTES == int(m.group(1)) << int(m.group(2))
    m = re.search(r"RECORD_SUMS_MAX\s*=\s*(\d+)\s*<<\s*(\d+)", hdr)
    assert m and bench.RECORD_SUMS_MAX == int(m.group(1)) << int(m.group(2))
    assert "return (int64_t)(sh.E + 2 * sh.N + 2) * sh.N <= RECORD_SUMS_MAX;" in hdr
    assert "if (!pack_in_row_order(sh))\n        return sh.partial || !sh.fixed;" in hdr
    assert "return sh.partial && !record_sums(sh);" in hdr
    c = CONFIGS["C"]
    small, big = c, c.with_(T=256)           # 1.75 MiB and 3.5 MiB per sender
    # 128 ranks x 256 experts: (256 + 2*128 + 2) * 128 = 65 792 terms per
    # record block, past the limit (DeepSeek-R1 decode: 10 304)
    wide = c.with_(N=128, T=8)
    base = bench.kernel_bytes(small, layout="fixed")["route_plan"]
    for cfg, transport, combine, layout, tail in [
            (small, "staged", "receiver", "packed", False), (small, "direct", "receiver", "packed", False),
            (small, "staged", "receiver", "fixed", False), (small, "staged", "partial", "packed", False),
            (small, "direct", "partial", "fixed", False), (wide, "staged", "partial", "packed", True),
            (wide, "staged", "receiver", "packed", False),
            (big, "staged", "receiver", "packed", True), (big, "direct", "receiver", "packed", True),
            (big, "staged", "receiver", "fixed", False), (big, "staged", "partial", "fixed", True)]:
        assert bench.plan_forms_offsets(cfg, combine, layout) == tail
        kb = bench.kernel_bytes(cfg, transport, combine, 1000 if combine == "partial" else 0, layout)
        R, N, E = cfg.rows, cfg.N, cfg.E
        offs = 4 * (N * E + N * (E + 1) + N * (N + 1) + (N + 1) + (E + 1))
        plain = 4 * (2 * R + N * E + 2 * N * (E + 1)) + (4 * R if cfg is not big else 0)
        extra = kb["route_plan"] - plain
        maps = kb["recv_map"] - offs - R * (24 if layout == "fixed" else 20)
        if combine == "partial":
            extra -= 2 * R * 4 + 2 * N * (N + 1) * 4
            if tail:
                extra -= N * (E + 2 * N + 2) * 4 + 2 * N * (N + 1) * 4 + 2 * (N + 1) * 4
            else:
                maps -= N * (N + 1) * 4 + 2 * (N + 1) * 4
        assert extra == (offs if tail else 0), (cfg.N, cfg.T, transport, combine, layout)
        assert maps == 0, (cfg.N, cfg.T, transport, combine, layout)
    assert base == 4 * (3 * c.rows + c.N * c.E + 2 * c.N * (c.E + 1))


def test_partial_byte_model_moves_p_rows():
    """With the partial combine the combine passes carry P rows instead of R."""
    cfg = CONFIGS["C"]
    P = 29_804
    kb = bench.kernel_bytes(cfg, "staged", "partial", P)
    hy = 2 * cfg.H
    assert kb["partial_transfer"] == 2 * P * hy
    # every expert row read once with its weight, one 32-byte record per
    # partial row
    assert kb["partial_send"] - P * hy == cfg.rows * (hy + 4) + P * 32
    assert kb["partial_reduce"] - P * hy == cfg.rows * 8 + cfg.N * cfg.T * cfg.H * 2
    assert "combine_reduce" not in kb and "transfer_back" not in kb


@pytest.mark.parametrize("key", ["A", "B", "E"])
def test_partial_rows_brute_force(key):
    cfg = CONFIGS[key].with_(T=min(CONFIGS[key].T, 24))
    idx = make_routing(cfg)[0]
    pairs = set()
    for s in range(cfg.N):
        for t in range(cfg.T):
            for k in range(cfg.K):
                pairs.add((s, t, int(idx[s, t, k]) // cfg.L))
    assert bench.partial_rows(cfg, idx) == len(pairs)


def test_code_only_ignores_comments_keeps_strings():
    a = 'int x = 1; // note\n/* block\n comment */ const char* s = "// not a comment";\n'
    b = 'int x = 1;\nconst char* s = "// not a comment";'
    assert bench._code_only(a) == bench._code_only(b)
    assert '"// not a comment"' in bench._code_only(a)
    assert bench._code_only("a  b\n\tc") == "a b c"
    assert bench._code_only("x = 1; // a") != bench._code_only("x = 2; // a")


def _counters_db(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (kernel_name text, counter_name text, value real)")
    con.executemany("insert into counters_collection values (?, ?, ?)", rows)
    con.commit()
    con.close()


def test_traffic_scaling_from_counters(tmp_path):
    """Each counter is scaled by CAL_BYTES / (its reading on the calibration
    copy): a kernel that reads what the copy read moves CAL_BYTES."""
    cfg = CONFIGS["C"]
    cal = bench.CAL_BYTES
    copy_name = "void at::native::elementwise_kernel<128, 4>(int, Func)"
    tr = "void moe::(anonymous namespace)::transfer_kernel<4, 4>(moe::Shape, ...)"
    # the counters see half the fetched bytes and all the written bytes
    _counters_db(tmp_path / "cal_f.db", [(copy_name, "FETCH_SIZE", cal / 2048.0)] * 5)
    _counters_db(tmp_path / "cal_w.db", [(copy_name, "WRITE_SIZE", cal / 1024.0)] * 5)
    kb = bench.kernel_bytes(cfg)["transfer"]
    half = kb / 2
    _counters_db(tmp_path / "f.db", [(tr, "FETCH_SIZE", half / 2048.0)] * 3)
    _counters_db(tmp_path / "w.db", [(tr, "WRITE_SIZE", half / 1024.0)] * 3)
    rec = bench.traffic_from(cfg, str(tmp_path / "f.db"), str(tmp_path / "w.db"),
                             str(tmp_path / "cal_f.db"), str(tmp_path / "cal_w.db"))
    assert rec["fetch_factor"] == 2.0 and rec["write_factor"] == 1.0
    t = rec["kernels"]["transfer"]
    assert t["launches"] == 3
    assert abs(t["hbm_bytes_per_launch"] - kb) <= 2
    assert t["ratio"] == 1.0
    assert rec["source_hash"] == bench.kernel_source_hash()


def test_trace_summary_table(tmp_path):
    cfg = CONFIGS["C"]
    db = tmp_path / "trace.db"
    con = sqlite3.connect(db)
    con.execute("create table kernels (name text, start integer, duration integer)")
    rows = [("void moe::(anonymous namespace)::transfer_kernel<4, 4>(...)", i, d)
            for i, d in enumerate((150_000, 160_000, 170_000))]
    rows += [("void moe::(anonymous namespace)::route_plan_kernel(moe::RouteArgs, moe::Plan)", 9,
              12_000)]
    rows += [("void at::native::vectorized_elementwise_kernel<4>(...)", 10, 5_000)]
    con.executemany("insert into kernels values (?, ?, ?)", rows)
    con.commit()
    con.close()
    table = bench.trace_summary(cfg, str(db)).splitlines()
    assert table[0].startswith("| kernel | launches | avg us")
    body = {line.split("|")[1].strip(): line for line in table[2:]}
    assert set(body) == {"route_plan", "transfer"}
    cells = [c.strip() for c in body["transfer"].split("|")[1:-1]]
    assert cells[1:5] == ["3", "160.00", "150.00", "170.00"]
    kb = bench.kernel_bytes(cfg)["transfer"]
    assert int(cells[5]) == round(kb / 160e-6 / 1e9)


def test_several_gpus_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_workload_named_or_unknown():
    """--config takes a workload's key or its name; an unknown one is refused."""
    bench_py = os.path.join(ROOT, "bench.py")
    r = subprocess.run([sys.executable, bench_py, "--config", "deepseek-r1-decode", "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr       # the name resolved
    r = subprocess.run([sys.executable, bench_py, "--config", "no-such-workload"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "unknown workload" in r.stderr and r.stdout == ""


def test_traffic_summary_names():
    """Each workload and mode has its own counter summary; the fixed-slot
    layout does not read the packed layout's."""
    import argparse
    key = lambda **kw: bench.traffic_key(argparse.Namespace(**kw))  # noqa: E731
    assert key(config="C", transport="staged", combine="receiver", layout="packed") == "C"
    assert key(config="C", transport="direct", combine="partial", layout="packed") == \
        "C_direct_partial"
    assert key(config="D", transport="staged", combine="receiver", layout="fixed") == "D_fixed"
    h = bench.kernel_source_hash()
    assert bench.measured_traffic("C_fixed", "transfer", h) is None


def test_trace_summary_timed_region(tmp_path):
    """The timed-region column averages each kernel's launches after the
    first cycle, the warmup, the all-kernel timing pass and the warm leg."""
    cfg = CONFIGS["C"]
    db = tmp_path / "trace.db"
    con = sqlite3.connect(db)
    con.execute("create table kernels (name text, start integer, duration integer)")
    steps, warmup = 3, 2
    first = 1 + warmup + 10 + steps
    durs = [100_000] * first + [200_000, 210_000, 220_000] + [100_000] * steps
    name = "void moe::(anonymous namespace)::transfer_kernel<4, 4>(...)"
    con.executemany("insert into kernels values (?, ?, ?)",
                    [(name, 1000 - i, d) for i, d in enumerate(reversed(durs))])
    con.commit()
    con.close()
    table = bench.trace_summary(cfg, str(db), (steps, warmup)).splitlines()
    assert table[0].endswith("timed-region avg us |")
    cells = [c.strip() for c in table[2].split("|")[1:-1]]
    assert cells[0] == "transfer" and cells[-1] == "210.00"


def test_traffic_cross_check_from_request_counters(tmp_path):
    """The DRAM-request bytes per request and the EA-request factors come from
    the calibration copy; a kernel whose requests match the copy's moves the
    copy's bytes."""
    cfg = CONFIGS["C"]
    cal = bench.CAL_BYTES
    copy_name = "void at::native::elementwise_kernel<128, 4>(int, Func)"
    tr = "void moe::(anonymous namespace)::transfer_kernel<4, 4>(moe::Shape, ...)"
    # the copy: 128-byte DRAM reads, 64-byte DRAM writes; EA reads of 128 B
    # counted as 64 by the formula, 64-byte EA writes
    _counters_db(tmp_path / "cal_d.db", [(copy_name, "TCC_EA0_RDREQ_DRAM_sum", cal / 128),
                                         (copy_name, "TCC_EA0_WRREQ_DRAM_sum", cal / 64)] * 5)
    _counters_db(tmp_path / "cal_q.db", [(copy_name, "TCC_EA0_RDREQ_sum", cal / 128),
                                         (copy_name, "TCC_EA0_RDREQ_32B_sum", 0),
                                         (copy_name, "TCC_EA0_WRREQ_sum", cal / 64),
                                         (copy_name, "TCC_EA0_WRREQ_64B_sum", cal / 64)] * 5)
    _counters_db(tmp_path / "d.db", [(tr, "TCC_EA0_RDREQ_DRAM_sum", cal / 128),
                                     (tr, "TCC_EA0_WRREQ_DRAM_sum", cal / 64)] * 3)
    _counters_db(tmp_path / "q.db", [(tr, "TCC_EA0_RDREQ_sum", cal / 128),
                                     (tr, "TCC_EA0_RDREQ_32B_sum", 0),
                                     (tr, "TCC_EA0_WRREQ_sum", cal / 64),
                                     (tr, "TCC_EA0_WRREQ_64B_sum", cal / 64)] * 3)
    tj = tmp_path / "traffic.json"
    tj.write_text(json.dumps({"kernels": {"transfer": {"hbm_bytes_per_launch": 2 * cal}}}))
    rec = bench.traffic_xcheck(cfg, str(tmp_path / "d.db"), str(tmp_path / "cal_d.db"),
                               str(tmp_path / "q.db"), str(tmp_path / "cal_q.db"), str(tj))
    assert rec["bytes_per_dram_read_request"] == 128.0
    assert rec["bytes_per_dram_write_request"] == 64.0
    assert rec["ea_read_factor"] == 2.0 and rec["ea_write_factor"] == 1.0
    t = rec["kernels"]["transfer"]
    assert t["dram_requests"] == 2 * cal and t["ea_requests"] == 2 * cal
    assert t["dram_over_fetch_write"] == 1.0 and t["ea_over_fetch_write"] == 1.0
