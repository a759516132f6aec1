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
    table = ("| shape | sizes | kernel us | HBM read bytes | HBM write bytes | x |\n|---|---|---|---|---|---|\n"
             "| c2 | g=2 | 26.1 (25.9) | 1,000 | 24 | 1.4x |\n| c4 | g=8 | 97.2 (97.2) | 2,000,000 | 8 | 1.4x |\n")
    shapes = os.path.join(tmp_path, "shapes.md")
    c1 = os.path.join(tmp_path, "c1.md")
    _write(shapes, f"kernel_source_sha256_16: {h}\n\n" + table)
    _write(c1, f"kernel_source_sha256_16: {h}\ntraffic_bytes_per_launch: 777\n")
    monkeypatch.setattr(bench, "SHAPES_PROFILE", shapes)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", c1)
    assert bench.recorded_shape_traffic() == {"c1": 777.0, "c2": 1024.0, "c4": 2_000_008.0}
    # a summary taken on another kernel source is not used
    _write(shapes, "kernel_source_sha256_16: 0000000000000000\n\n" + table)
    _write(c1, "kernel_source_sha256_16: 0000000000000000\ntraffic_bytes_per_launch: 777\n")
    assert bench.recorded_shape_traffic() == {}
