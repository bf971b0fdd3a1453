"""Host logic of the rocprofv3 summariser: HBM bytes per dispatch scaled by the reading of a copy
of known size, and the marker filter that keeps only the dispatches after the last marker kernel
(so a prefill before the timed steps is left out)."""
import csv

from rq_transformer_frame_amd import profsum

COLS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def write_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COLS)
        w.writeheader()
        for i, (name, v) in enumerate(rows, 1):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": v})


def test_traffic_scales_by_the_copy_and_filters_after_marker(tmp_path):
    # a 1 MiB copy whose FETCH_SIZE reads half its size (scale 2) and WRITE_SIZE its size (scale 1)
    seq = [("__amd_rocclr_copyBuffer", None), ("mk::k_prefill_ring", None), ("attn_kernel", None),
           ("mk::k_prefill_ring", None), ("attn_kernel", None), ("attn_kernel", None)]
    fetch = [512.0, 1.0, 1000.0, 1.0, 10.0, 30.0]
    write = [1024.0, 1.0, 500.0, 1.0, 4.0, 4.0]
    fp, wp = tmp_path / "f.csv", tmp_path / "w.csv"
    write_csv(fp, "FETCH_SIZE", [(n, v) for (n, _), v in zip(seq, fetch)])
    write_csv(wp, "WRITE_SIZE", [(n, v) for (n, _), v in zip(seq, write)])

    def row(text, name):
        return next(line for line in text.splitlines() if line.startswith(f"| {name} "))

    every = profsum.traffic(str(fp), str(wp), 1.0)
    assert "FETCH_SIZE x 2.000, WRITE_SIZE x 1.000" in every
    # all three attention dispatches: fetch mean 1040/3 KiB x 2, write mean 508/3 KiB
    cells = row(every, "attn_kernel").split("|")
    assert cells[2].strip() == "3"
    assert int(cells[5]) == round((1040 / 3 * 2 + 508 / 3) * 1024)
    after = profsum.traffic(str(fp), str(wp), 1.0, "k_prefill_ring")
    cells = row(after, "attn_kernel").split("|")
    assert cells[2].strip() == "2"
    assert int(cells[5]) == round((20 * 2 + 4) * 1024)
    assert "k_prefill_ring" not in after.split("| stage")[1].split("\n", 2)[2]


def test_phase_kinds_of_the_persistent_frame():
    # 32 temporal layers x 5 phases, the text head, then 8 codebook steps of 6 layers x 4 phases
    # and a head: 32 * 5 + 1 + 8 * 25 = 361 phases
    from collections import Counter

    from rq_transformer_frame_amd.phase_timeline import phase_kind
    kinds = [phase_kind(p, 32, 6) for p in range(361)]
    c = Counter(kinds)
    assert [c[k] for k in ("qkv", "attention", "out_proj", "gate_in", "gate_out")] == [32] * 5
    assert c["text_head+dep_in"] == 1 and kinds[160] == "text_head+dep_in"
    assert [c[k] for k in ("dep_qkv", "dep_attention+out_proj", "dep_gate_in", "dep_gate_out")] == [48] * 4
    assert c["dep_head"] == 8 and kinds[360] == "dep_head" and kinds[185] == "dep_head"
    assert kinds[161] == "dep_qkv" and kinds[186] == "dep_qkv"
