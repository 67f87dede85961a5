"""Host logic of the counter summary: per-launch traffic from two counter runs
scaled by the calibration dispatches."""
import csv
import json

from symmetric_nmf_clustering_amd import profile_passes as pp

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
SH = "void symnmf::sh_panel_kernel<1, 8, 2, true, 0>(float const*, long, float const*, int, symnmf::RowPlan, int, float*, int)"
SAMPLED = SH.replace(", 0>(", ", 1>(")
MUL = "void at::native::elementwise_kernel<128, 4, MulFunctor<float>>(int, ...)"


def _write(tmp_path, name, counter, rows, copy_bytes):
    path = tmp_path / f"{name}.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (kern, val) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": kern, "Counter_Name": counter,
                        "Counter_Value": val})
    jpath = tmp_path / f"{name}.json"
    jpath.write_text("noise line\n" + json.dumps({"n": 1000, "k": 24, "copy_bytes_each_way": copy_bytes,
                                                   "copy_reps": 3}) + "\n")
    return str(path), str(jpath)


def test_summary_scales_by_calibration(tmp_path):
    cb = 1 << 30
    # read counter reports half the bytes (factor 2); write counter is exact
    f_csv, f_json = _write(tmp_path, "fetch", "FETCH_SIZE",
                           [(SH, 100.0), (SAMPLED, 5.0), (SH, 300.0)] + [(MUL, cb / 1024 / 2)] * 3, cb)
    w_csv, w_json = _write(tmp_path, "write", "WRITE_SIZE",
                           [(SH, 10.0), (SH, 30.0)] + [(MUL, cb / 1024)] * 3, cb)
    out = tmp_path / "out.json"
    pp.summarize(["--fetch-csv", f_csv, "--fetch-json", f_json, "--write-csv", w_csv,
                  "--write-json", w_json, "--out", str(out)])
    rec = json.load(open(out))
    assert rec["fetch_size_factor"] == 2.0 and rec["write_size_factor"] == 1.0
    assert rec["fetch_size_launches"] == 2  # the sampled pass is not a full pass
    assert rec["traffic_bytes_per_launch"] == 200.0 * 1024 * 2 + 20.0 * 1024
    assert rec["algorithmic_bytes_per_launch"] == 4.0 * 1000 * 1000 + 8.0 * 1000 * 24
    assert rec["kernel"] == "sh_panel_kernel<1, 8, 2, true, 0>"
    assert len(rec["source_sha256"]) == 64
