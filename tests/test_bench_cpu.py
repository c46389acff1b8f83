"""Host-side logic of bench.py: the traffic figure is tied to the sources of
the kernels it was measured on."""
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_every_csrc_kernel_file_is_mapped():
    csrc = os.path.join(ROOT, "block_scaled_fp8_linear_amd", "csrc")
    mapped = set(bench.SHARED_SOURCES)
    for files in bench.KERNEL_SOURCES.values():
        mapped.update(files)
    assert set(os.listdir(csrc)) - mapped == set(), "a source file belongs to no kernel"
    for name in mapped:
        assert os.path.exists(os.path.join(csrc, name)), name


def test_source_sha_depends_only_on_the_kernels_files():
    real = lambda name: open(os.path.join(ROOT, "block_scaled_fp8_linear_amd", "csrc", name), "rb").read()
    edited = lambda name: real(name) + (b"static int edit_marker;\n" if name == "gemm_w8a8.hip" else b"")
    tiled = ["gemm_tiled_kernel<128, 128, 2>", "reduce_partials_kernel"]
    w8 = ["gemm_w8a8_kernel", "act_quantize_kernel"]
    assert bench.kernel_source_sha(tiled, read=real) == bench.kernel_source_sha(tiled, read=edited)
    assert bench.kernel_source_sha(w8, read=real) != bench.kernel_source_sha(w8, read=edited)
    # template arguments do not matter, the kernel does
    assert bench.kernel_source_sha(["gemm_tiled_kernel<256, 128, 2>"], read=real) == \
        bench.kernel_source_sha(["gemm_tiled_kernel<128, 256, 2>"], read=real)
    with pytest.raises(KeyError):
        bench.kernel_source_sha(["some_other_kernel"], read=real)


def test_source_sha_ignores_comments_only():
    real = lambda name: open(os.path.join(ROOT, "block_scaled_fp8_linear_amd", "csrc", name), "rb").read()
    tiled = ["gemm_tiled_kernel<128, 128, 2>"]
    base = bench.kernel_source_sha(tiled, read=real)

    def commented(name):
        src = real(name)
        if name != "gemm_tiled.hip":
            return src
        # a new comment line, a reworded block comment, a trailing comment
        return (b"// note\n" + src.replace(b"namespace fp8bl {", b"namespace fp8bl {  /* x */", 1)
                + b"\n\n// end\n")

    def recoded(name):
        src = real(name)
        return src.replace(b"constexpr int kBK = 64;", b"constexpr int kBK = 32;", 1) \
            if name == "gemm_tiled.hip" else src

    assert b"constexpr int kBK = 64;" in real("gemm_tiled.hip")
    assert bench.kernel_source_sha(tiled, read=commented) == base
    assert bench.kernel_source_sha(tiled, read=recoded) != base
    # comment markers inside literals are code
    assert bench.code_only(b'const char* s = "// x";\n') == b'const char* s = "// x";'
    assert bench.code_only(b"char c = '/'; // y\nint z;\n") == b"char c = '/';\nint z;"


def test_measured_traffic_follows_the_recorded_sha(tmp_path, monkeypatch):
    data = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    for w, ent in data["workloads"].items():
        v = bench.measured_traffic(w)
        assert v is None or (v == ent["hbm_bytes_per_launch"] and
                             ent["source_sha"] == bench.kernel_source_sha(ent["kernels"]))
    # a fresh entry reads back, a stale one reads as null
    os.symlink(os.path.join(ROOT, "block_scaled_fp8_linear_amd"), tmp_path / "block_scaled_fp8_linear_amd")
    prof = tmp_path / "profiles"
    prof.mkdir()
    good = {"hbm_bytes_per_launch": 123, "kernels": ["dequant_kernel"],
            "source_sha": bench.kernel_source_sha(["dequant_kernel"])}
    stale = dict(good, source_sha="0" * 16)
    (prof / "traffic.json").write_text(json.dumps({"workloads": {"good": good, "stale": stale}}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("good") == 123
    assert bench.measured_traffic("stale") is None
    assert bench.measured_traffic("absent") is None
