"""Host-side checks of the built library's gfx950 code objects (no GPU needed).

A kernel that keeps arrays in private (scratch) memory runs several times
slower than its register-resident form: a block routine that the compiler
declines to inline, or a launch bound that forces registers out, does that
without any compile error.  The device code of libnsa.so is read back from
its offload bundles and every kernel's private segment is checked against a
small bound (a few spilled registers outside the hot loops are tolerated)."""
import os
import re
import subprocess

import pytest

import sparse_attention_long_compress_amd as nsa

LLVM = "/opt/rocm/llvm/bin"
MAX_PRIVATE_BYTES = 64
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def kernel_private_segments(lib_path, tmp_path):
    fatbin = tmp_path / "fatbin"
    subprocess.run([f"{LLVM}/llvm-objcopy", f"--dump-section=.hip_fatbin={fatbin}", lib_path,
                    str(tmp_path / "host_copy")], check=True, capture_output=True)
    data = fatbin.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    out = {}
    for i, st in enumerate(starts):
        part = tmp_path / f"bundle{i}"
        part.write_bytes(data[st:starts[i + 1] if i + 1 < len(starts) else len(data)])
        co = tmp_path / f"gfx950_{i}.co"
        subprocess.run([f"{LLVM}/clang-offload-bundler", "--unbundle", "--type=o",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--input={part}",
                        f"--output={co}"], check=True, capture_output=True)
        notes = subprocess.run([f"{LLVM}/llvm-readelf", "--notes", str(co)], check=True,
                               capture_output=True, text=True).stdout
        for m in re.finditer(r"\.name:\s+(\S+)\s*\n(?:.*\n)*?\s*\.private_segment_fixed_size:\s+(\d+)",
                             notes):
            out[m.group(1)] = int(m.group(2))
    return out


@pytest.mark.skipif(not os.path.exists(os.path.join(LLVM, "clang-offload-bundler")),
                    reason="ROCm LLVM tools not installed")
def test_no_kernel_keeps_arrays_in_scratch(tmp_path):
    lib_path = nsa.LIB_PATH
    if not os.path.exists(lib_path):
        pytest.skip("libnsa.so is not built")
    seg = kernel_private_segments(lib_path, tmp_path)
    # every kernel family of the library is present
    for family in ("pool_kernel", "cmp_select_kernel", "sel_win_kernel", "sel_compact_kernel",
                   "bwd_dq_kernel", "bwd_dkdv_kernel", "decode_mfma_kernel", "decode_kernel"):
        assert any(family in k for k in seg), family
    big = {k: v for k, v in seg.items() if v > MAX_PRIVATE_BYTES}
    assert not big, big
