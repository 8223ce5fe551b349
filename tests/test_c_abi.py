"""The C ABI from plain C, without a GPU: tests/c/abi_check.c is compiled with gcc against
include/veda.h and linked against the built libveda.so; its answers are checked here."""
import os
import shutil
import subprocess

import pytest

from conftest import gpu_visible

pytestmark = pytest.mark.skipif(gpu_visible(), reason="fake device addresses: CPU-only (no GPU visible)")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "video_dit_block_head_amd")
ROCM_INC = "/opt/rocm/include"


@pytest.fixture(scope="module")
def c_out(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not available")
    if not os.path.exists(os.path.join(LIB_DIR, "libveda.so")):
        pytest.skip("libveda.so is not built")
    if not os.path.isdir(ROCM_INC):
        pytest.skip("ROCm headers are not available")
    exe = str(tmp_path_factory.mktemp("cabi") / "abi_check")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror=implicit-function-declaration",
                    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", ROCM_INC,
                    os.path.join(ROOT, "tests", "c", "abi_check.c"), "-o", exe, "-L", LIB_DIR, "-lveda",
                    f"-Wl,-rpath,{LIB_DIR}"], check=True, capture_output=True, text=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    return dict(line.split(" ", 1) for line in out.strip().splitlines())


def test_version_and_status(c_out):
    assert "gfx950" in c_out["version"]
    assert c_out["status_null"]


def test_sizes(c_out):
    # the large workload: 600 tiles of 128 tokens per head, every shape dividing the grid
    assert int(c_out["tiled_tokens"]) == 76800
    assert int(c_out["head_tiles_0"]) == 600
    assert int(c_out["tilemap_ws_64"]) > 0
    # the estimator outputs y_q, y_k [2][B][H][n_t][64] fp32, rounded up to 256 bytes
    assert int(c_out["trippool_ws"]) == 2 * 40 * 600 * 64 * 4


def test_validation(c_out):
    assert int(c_out["attn_null"]) == -1      # VEDA_ERR_NULL
    assert int(c_out["attn_dtype"]) == -3     # VEDA_ERR_DTYPE
    assert int(c_out["attn_v_raster"]) == -4  # VEDA_ERR_UNSUPPORTED: a raster V needs the raster call
    assert int(c_out["topk_k0"]) == -2        # VEDA_ERR_SHAPE
    assert int(c_out["topk_empty"]) == 0      # zero rows: nothing to do
    assert int(c_out["tiled_tokens_bad"]) == -2


def test_readme_c_example_compiles(tmp_path):
    """The C example of README.md (the default step through include/veda.h) compiles against
    the header as it stands, warnings as errors."""
    if shutil.which("gcc") is None or not os.path.isdir(ROCM_INC):
        pytest.skip("gcc or the ROCm headers are not available")
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = text.split("```c\n")[1:]
    assert blocks, "README.md has no C example"
    src = tmp_path / "readme_step.c"
    src.write_text(blocks[0].split("```")[0])
    subprocess.run(["gcc", "-c", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", ROCM_INC, str(src), "-o", str(tmp_path / "s.o")],
                   check=True, capture_output=True, text=True)
