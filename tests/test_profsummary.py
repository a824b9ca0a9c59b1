"""Host logic of the rocprofv3 summaries: the launch-set mapping of
profsummary `sets` on small synthetic result databases of the same schema."""
import json
import sqlite3

from quantized_bit_gemm_amd import profsummary

GEMM = "void qbg::(anonymous namespace)::gemm_lds_kernel<0, true, 32>(qbg::GemmArgs)"
COPY = "__amd_rocclr_copyBuffer"


def _trace_db(path, durations_ns):
    c = sqlite3.connect(path)
    c.execute("create table kernels (name text, start integer, duration integer)")
    t = 0
    c.execute("insert into kernels values (?, ?, ?)", (COPY, t, 1000))
    for d in durations_ns:
        t += 10000
        c.execute("insert into kernels values (?, ?, ?)", (GEMM, t, d))
        c.execute("insert into kernels values (?, ?, ?)", ("fill_kernel", t + 1, 5))
    c.commit()


def _pmc_db(path, counter, copy_raw, values):
    c = sqlite3.connect(path)
    c.execute("create table counters_collection (kernel_name text, dispatch_id integer, "
              "counter_name text, value real)")
    c.execute("insert into counters_collection values (?, ?, ?, ?)", (COPY, 1, counter, copy_raw))
    for i, v in enumerate(values):
        # two rows for one dispatch: the summary adds them
        c.execute("insert into counters_collection values (?, ?, ?, ?)", (GEMM, 10 + i, counter, v / 2))
        c.execute("insert into counters_collection values (?, ?, ?, ?)", (GEMM, 10 + i, counter, v / 2))
    c.commit()


def test_sets_summary_maps_dispatches_to_entries(tmp_path):
    sets = []
    for M in (1, 32):
        e = {"op": "fp8", "N": 4096, "K": 4096, "M": M}
        sets.append(dict(e, role="winner", config={"kernel_id": 16, "swap_ab": 1, "split_k": 2,
                                                   "rotate": 0}, select_us=5.0))
        sets.append(dict(e, role="runner-up", config={"kernel_id": 4, "swap_ab": 0, "split_k": 4,
                                                      "rotate": 0}, select_us=6.0))
    sp = tmp_path / "sets.json"
    sp.write_text(json.dumps(sets))
    reps = 3
    # set i has durations (i+1) us each; fetch (i+1) * 1000 raw KiB
    durs = [(i + 1) * 1000 for i in range(4) for _ in range(reps)]
    _trace_db(str(tmp_path / "t.db"), durs)
    # calibration copy of 1 MiB reads 512 raw KiB: scale 2
    _pmc_db(str(tmp_path / "f.db"), "FETCH_SIZE", 512.0,
            [(i + 1) * 1000.0 for i in range(4) for _ in range(reps)])
    rows, scales = profsummary.sets_summary(str(sp), str(tmp_path / "t.db"), [str(tmp_path / "f.db")],
                                            reps, 1)
    assert scales == {"FETCH_SIZE": 2.0}
    assert [round(r["us"], 6) for r in rows] == [1.0, 2.0, 3.0, 4.0]
    assert [round(r["counters"]["FETCH_SIZE_MB"], 6) for r in rows] == [
        round((i + 1) * 1000 * 2 * 1024 / 1e6, 6) for i in range(4)]
    text = "\n".join(profsummary.render_sets(rows, scales, ["cmd"]))
    assert "entries: 2; winner faster in the kernel trace: 2" in text
    assert "16/1/2" in text and "4/0/4" in text


def test_sets_summary_rejects_a_dispatch_count_mismatch(tmp_path):
    sp = tmp_path / "sets.json"
    sp.write_text(json.dumps([{"op": "fp8", "N": 16, "K": 16, "M": 1, "role": "case",
                               "config": {"kernel_id": 0, "swap_ab": 0, "split_k": 1}}]))
    _trace_db(str(tmp_path / "t.db"), [1000] * 4)
    try:
        profsummary.sets_summary(str(sp), str(tmp_path / "t.db"), [], 3, 1)
    except SystemExit as e:
        assert "expected 3 GEMM dispatches" in str(e)
    else:
        raise AssertionError("a mismatch must be reported")


def test_sets_summary_drops_the_warmup_dispatches(tmp_path):
    sp = tmp_path / "sets.json"
    sp.write_text(json.dumps([{"op": "fp8", "N": 16, "K": 16, "M": 1, "role": "case",
                               "config": {"kernel_id": 0, "swap_ab": 0, "split_k": 1}}] * 2))
    # per set: 2 warmup dispatches of 100 us, then 3 of (set + 1) us
    durs = [100000, 100000, 1000, 1000, 1000, 100000, 100000, 2000, 2000, 2000]
    _trace_db(str(tmp_path / "t.db"), durs)
    rows, _ = profsummary.sets_summary(str(sp), str(tmp_path / "t.db"), [], 3, 1, warmup=2)
    assert [round(r["us"], 6) for r in rows] == [1.0, 2.0]
