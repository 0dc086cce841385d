"""The built library's gfx950 kernels need no scratch memory.

A kernel with a private segment (a call stack, spilled vector registers) makes the
GPU set up scratch for every dispatch, which costs microseconds per launch --
the exchange is a few-microsecond kernel, so that alone would show up as a
large slowdown.  This reads the kernel descriptors' metadata from the code
object that libhr.so carries (our own build) with the ROCm LLVM tools and
checks every kernel.  CPU only.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "message_fp16_all_amd", "libhr.so")
LLVM = "/opt/rocm/llvm/bin"


MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def kernel_metadata(tmp_path):
    """Kernel name -> scratch-related metadata, over every translation unit's
    bundle in the library's .hip_fatbin section."""
    fatbin = tmp_path / "fatbin.bin"
    subprocess.run([f"{LLVM}/llvm-objcopy", f"--dump-section=.hip_fatbin={fatbin}", LIB,
                    str(tmp_path / "lib.copy")], check=True)
    data = fatbin.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    notes = ""
    for i, st in enumerate(starts):
        chunk = tmp_path / f"bundle{i}.bin"
        co = tmp_path / f"co{i}.o"
        chunk.write_bytes(data[st:starts[i + 1] if i + 1 < len(starts) else len(data)])
        subprocess.run([f"{LLVM}/clang-offload-bundler", "--type=o",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--input={chunk}",
                        f"--output={co}", "--unbundle"], check=True)
        notes += subprocess.run([f"{LLVM}/llvm-readelf", "--notes", str(co)], check=True,
                                capture_output=True, text=True).stdout
    kernels = {}
    name = None
    for line in notes.splitlines():
        m = re.match(r"\s+\.name:\s+(\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.match(r"\s+\.(private_segment_fixed_size|uses_dynamic_stack|vgpr_spill_count|"
                     r"sgpr_spill_count):\s+(\S+)", line)
        if m and name is not None:
            kernels[name][m.group(1)] = m.group(2)
    return kernels


@pytest.mark.skipif(not os.path.exists(LIB) or not os.path.exists(f"{LLVM}/llvm-readelf"),
                    reason="libhr.so not built or ROCm LLVM tools missing")
def test_no_kernel_uses_scratch(tmp_path):
    kernels = kernel_metadata(tmp_path)
    assert any("exchange_k" in k for k in kernels) and any("fold_vec" in k for k in kernels)
    # a VGPR spill or a call stack needs scratch memory; an SGPR spill goes
    # to a VGPR lane (and would show a private segment if it did not)
    bad = {k: v for k, v in kernels.items()
           if v.get("private_segment_fixed_size", "0") != "0"
           or v.get("uses_dynamic_stack", "false") != "false"
           or v.get("vgpr_spill_count", "0") != "0"}
    assert not bad, f"kernels with scratch: {sorted(bad)[:5]}"
