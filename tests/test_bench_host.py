"""Host logic of bench.py (CPU only): the algorithmic byte counts behind the
roofline, the name of the scan instantiation it reports (which must be the
kernel the committed profiles list), the code hash that keys the committed
traffic counters, and the single-GPU refusal."""

import os
import subprocess
import sys

import bench

HERE = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_scan_algorithmic_bytes():
    # 128 B per visible key + 4,224 B of query and weights per query
    assert bench.scan_algorithmic_bytes(8, 1, 8 * (1 << 20)) == 1073775616
    assert bench.scan_algorithmic_bytes(8, 1, 8 * (1 << 20), "fp4") == 570459136
    assert bench.scan_algorithmic_bytes(64, 1, 64 * (1 << 19)) == 128 * 64 * (1 << 19) + 64 * 4224
    # query tokens of one sequence share the key reads
    assert bench.scan_algorithmic_bytes(1, 16, 1000) == 128 * 1000 + 16 * 4224


def test_step_algorithmic_bytes_decoder_group():
    from synth.configs import WORKLOADS
    w = WORKLOADS["c2"]
    n_keys = w.B * w.n_cap
    full = 128 * n_keys + (4096 + 128 + 2048) * 8
    reindex = (16384 * 128 + 4224 + 8192 + 2048) * 8
    assert bench.step_algorithmic_bytes(w, n_keys) == full + 3 * reindex + 7 * 411648 * 8 + 1568 * 8


def test_scan_kernel_names_match_the_profiles():
    names = {
        "kernels_decoder_group_c2_1M_b8.md": bench.scan_kernel_name(0, 8, 1, 1 << 20),
        "kernels_decoder_group_c2_1M_b8_fp4k.md": bench.scan_kernel_name(1, 8, 1, 1 << 20),
        "kernels_encoder_group_c4_512k_b64.md": bench.scan_kernel_name(0, 64, 1, 1 << 19),
    }
    assert names["kernels_decoder_group_c2_1M_b8.md"] == "k_index_score_decode<0, 0, 1, 4>"
    assert names["kernels_encoder_group_c4_512k_b64.md"] == "k_index_score_decode<0, 0, 1, 8>"
    assert bench.scan_kernel_name(0, 8, 2, 1 << 20) == "k_index_score_decode<0, 0, 2, 8>"
    for f, name in names.items():
        with open(os.path.join(HERE, "profiles", f), encoding="utf-8") as fh:
            assert "| " + name + " |" in fh.read(), (f, name)


def test_source_hash_ignores_comments_and_blank_lines(tmp_path):
    code = "int a = 1;\nint b = a + 2;  \n"
    commented = "// header\n\nint a = 1;   // one\n\n// between\nint b = a + 2;\n"
    other = "int a = 1;\nint b = a + 3;\n"
    p1, p2, p3 = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    p1.write_text(code)
    p2.write_text(commented)
    p3.write_text(other)
    assert bench.source_sha(str(p1)) == bench.source_sha(str(p2))
    assert bench.source_sha(str(p1)) != bench.source_sha(str(p3))


def test_traffic_lookup_needs_the_same_algorithmic_bytes():
    # an entry is used only for the byte count it was measured at
    assert bench.read_traffic(12345) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(HERE, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=HERE, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
