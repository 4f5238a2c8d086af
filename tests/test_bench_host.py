"""Host-side checks of the benchmark's accounting (no GPU): the algorithmic
bytes per launch of each workload shape, which the reported GB/s and
roofline fractions are built on, and the one-GPU refusal."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_bytes_qwen3_8b_layer_and_step():
    # 13100 cells x 8 KV heads x (256 B K + 256 B V) + q and out (fp32, 32 heads x 128)
    per_layer = bench.algorithmic_bytes(13100, 8, 128, 0, 1, 32)
    assert per_layer == 13100 * 8 * 512 + 2 * 4 * 32 * 128 == 53690368
    assert 36 * per_layer == 1932853248


def test_bytes_long_context_layer():
    assert bench.algorithmic_bytes(524288, 8, 128, 0, 1, 40) == 2 * 2 ** 30 + 2 * 4 * 40 * 128 == 2147524608


@pytest.mark.parametrize("kind,want", [(1, 474096768), (2, 251494528)])
def test_bytes_gqa6_quantized(kind, want):
    # attended cells 131072 + 65536 + 20000 + 777; codes plus one f16 scale per
    # 32 elements for K and V; the 217600-entry compact plan; q and out of 4 slots
    cells = 131072 + 65536 + 20000 + 777
    assert bench.algorithmic_bytes(cells, 4, 256, kind, 4, 24, plan_entries=217600) == want


def test_bytes_mixed_kinds():
    cells = 131072 + 65536 + 20000 + 777
    row = (256 + 16) + (128 + 16)  # int8 K row + 4-bit V row, with their scales
    assert bench.algorithmic_bytes(cells, 4, 256, 1, 4, 24, plan_entries=217600, v_kind=2) == \
        cells * 4 * row + 4 * 217600 + 2 * 4 * 4 * 24 * 256


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in (r.stdout + r.stderr)


def test_kernel_hash_ignores_comments_only():
    src = 'int f(int x) {  // twice\n  return 2 * x; /* "doubled" */ }\nconst char* s = "a // b";\n'
    same = '// leading note\nint f(int x) {\n    return 2 * x;\n}\nconst char* s = "a // b";\n'
    other = 'int f(int x) { return 3 * x; }\nconst char* s = "a // b";\n'
    assert bench.strip_c_comments(src) == bench.strip_c_comments(same)
    assert bench.strip_c_comments(src) != bench.strip_c_comments(other)
    assert '"a // b"' in bench.strip_c_comments(src)


def test_bytes_single_layer_4096_and_rotation():
    # 4096 cells x 8 KV heads x 512 B + q and out; one launch per step over
    # 32 rotated copies (more than the 256 MB memory-side cache holds)
    wl = bench.WORKLOADS["single-4096"]()
    assert wl.algorithmic_bytes_per_launch() == 4096 * 8 * 512 + 2 * 4 * 32 * 128 == 16809984
    assert wl.layers // wl.cycle == 1
    assert wl.config()["rotated_bytes"] == 32 * 4096 * 8 * 128 * 4 > 256 * 2 ** 20


def test_library_hash_matches_sources():
    """The built library carries the hash of the sources beside it (a stale
    library is refused at import)."""
    from long_context_decode_kv_amd import build, kvdec
    assert kvdec.LIB_SOURCE_HASH == build.source_hash() == build.built_hash()
    assert len(kvdec.LIB_SOURCE_HASH) == 16
