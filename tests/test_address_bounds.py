"""Every global range the fused kernel's tile copies can read lies inside its
tensor, for ragged and tile-aligned lengths up to the longest accepted
sequence (host check, no GPU)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_tile_copies_stay_in_bounds(tmp_path):
    exe = str(tmp_path / "address_bounds")
    subprocess.run(["g++", "-O2", "-std=c++17", "-I",
                    os.path.join(ROOT, "gated_causal_attention_amd", "csrc"),
                    os.path.join(ROOT, "tests", "address_bounds.cpp"), "-o", exe], check=True)
    shapes = []
    for n in (1, 2, 31, 33, 63, 64, 65, 127, 128, 129, 191, 192, 200, 257, 383, 520, 1000):
        for d in (64, 128):
            shapes += [2, 2, n, d]
    shapes += [1, 1, 8192, 128, 1, 1, 32768, 128]
    shapes += [2, 8, 1000, 64]  # 16 heads: eight work queues of the bf16 forward
    shapes += [1, 1, 1 << 22, 128]  # the longest sequence the boundary accepts
    out = subprocess.run([exe, *map(str, shapes)], capture_output=True, text=True)
    print(out.stdout)
    assert out.returncode == 0, out.stdout
