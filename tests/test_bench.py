"""CPU checks of bench.py's host logic: algorithmic sizes of the page shapes and the reading of
the committed counter summaries (only when taken on the current kernel source)."""
import os

import bench


def test_algorithmic_sizes():
    # per-call bytes and flops of the four timed page shapes (each operand byte once, C once)
    assert bench.algorithmic_bytes([128, 384], 4096, 1536) == 11_714_560
    assert bench.algorithmic_bytes([192, 320], 3072, 4096) == 18_481_152
    assert bench.algorithmic_bytes([40, 76, 168, 72, 164, 148, 196, 160], 7168, 2048) == 81_920_000
    assert bench.algorithmic_bytes([80, 176, 128, 72, 64, 248, 96, 160], 4096, 7168) == 144_637_952
    assert bench.algorithmic_flops([128, 384], 4096, 1536) == 2 * 512 * 4096 * 1536


def _write(path, text):
    with open(path, "w") as f:
        f.write(text)


def test_shape_traffic_follows_the_kernel_source(tmp_path, monkeypatch):
    h = bench.kernel_source_hash()
    table = ("| shape | sizes | HBM read bytes | HBM write bytes | x |\n|---|---|---|---|---|\n"
             "| c2 | g=2 | 1,000 | 24 | 1.4x |\n| c4 | g=8 | 2,000,000 | 8 | 1.4x |\n")
    path = os.path.join(tmp_path, "traffic.md")
    _write(path, f"kernel_source_sha256_16: {h}\n\n" + table)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", path)
    assert bench.recorded_shape_traffic() == {"c2": 1024.0, "c4": 2_000_008.0}
    # a summary taken on another kernel source is not used
    _write(path, "kernel_source_sha256_16: 0000000000000000\n\n" + table)
    assert bench.recorded_shape_traffic() == {}


def test_cold_sequence_rotates_every_set():
    # the captured sequence of a replay covers all R sets whatever the step count is
    for name in ("c1", "c2", "c3", "c4"):
        cfg = bench.shape_of(name)
        nbytes = bench.algorithmic_bytes(cfg.m, cfg.n, cfg.k)
        for steps in (1, 20, 200):
            seq, R = bench.cold_sequence(steps, nbytes)
            assert R * nbytes >= bench.COLD_BYTES and (R - 1) * nbytes < bench.COLD_BYTES
            assert set(seq) == set(range(R)) and len(seq) == max(steps, R)
            assert all(seq[i + 1] != seq[i] for i in range(len(seq) - 1)) or R == 1
