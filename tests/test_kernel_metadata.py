"""Properties of the built library's gfx950 kernels, read from the code
object that libhr.so carries (our own build) with the ROCm LLVM tools.  CPU
only.

- No kernel needs scratch memory.  A kernel with a private segment (a call
  stack, spilled vector registers) makes the GPU set up scratch for every
  dispatch, which costs microseconds per launch -- the exchange is a
  few-microsecond kernel, so that alone would show up as a large slowdown.
- The per-rank exchange kernels receive their leading scalar arguments in
  SGPRs (kernel-argument preload), so that their first loads do not wait for
  a kernel-argument load.
"""
import struct
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "message_fp16_all_amd", "libhr.so")
LLVM = "/opt/rocm/llvm/bin"


MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def code_objects(tmp_path):
    """Paths of the gfx950 code objects, one per translation unit's bundle in
    the library's .hip_fatbin section."""
    fatbin = tmp_path / "fatbin.bin"
    subprocess.run([f"{LLVM}/llvm-objcopy", f"--dump-section=.hip_fatbin={fatbin}", LIB,
                    str(tmp_path / "lib.copy")], check=True)
    data = fatbin.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    paths = []
    for i, st in enumerate(starts):
        chunk = tmp_path / f"bundle{i}.bin"
        co = tmp_path / f"co{i}.o"
        chunk.write_bytes(data[st:starts[i + 1] if i + 1 < len(starts) else len(data)])
        subprocess.run([f"{LLVM}/clang-offload-bundler", "--type=o",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--input={chunk}",
                        f"--output={co}", "--unbundle"], check=True)
        paths.append(co)
    return paths


def kernel_descriptors(tmp_path):
    """Kernel symbol name -> its 64-byte kernel descriptor (the `<name>.kd`
    object), over every code object."""
    kds = {}
    for co in code_objects(tmp_path):
        sections = {}
        for line in subprocess.run([f"{LLVM}/llvm-readelf", "-S", "--wide", str(co)], check=True,
                                   capture_output=True, text=True).stdout.splitlines():
            m = re.match(r"\s*\[\s*(\d+)\]\s+(\S+)\s+\S+\s+([0-9a-f]+)\s+([0-9a-f]+)\s+([0-9a-f]+)", line)
            if m:
                sections[int(m.group(1))] = (int(m.group(3), 16), int(m.group(4), 16))
        blob = co.read_bytes()
        for line in subprocess.run([f"{LLVM}/llvm-readelf", "-s", "--wide", str(co)], check=True,
                                   capture_output=True, text=True).stdout.splitlines():
            f = line.split()
            if len(f) >= 8 and f[3] == "OBJECT" and f[7].endswith(".kd") and f[6].isdigit():
                addr, off = sections[int(f[6])]
                start = int(f[1], 16) - addr + off
                kds[f[7][:-3]] = blob[start:start + 64]
    return kds


def kernel_metadata(tmp_path):
    """Kernel name -> scratch-related metadata, over every code object."""
    notes = ""
    for co in code_objects(tmp_path):
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


@pytest.mark.skipif(not os.path.exists(LIB) or not os.path.exists(f"{LLVM}/llvm-readelf"),
                    reason="libhr.so not built or ROCm LLVM tools missing")
def test_per_rank_exchange_kernels_preload_their_leading_arguments(tmp_path):
    """The kernel descriptor's kernarg-preload field (bytes 58-59: the length
    in dwords in bits 0-6) shows 9 dwords, the five leading parameters (three
    pointers, numel, the active workgroup count), for every per-rank exchange
    kernel; the group kernels, whose first parameter is a struct, preload
    nothing."""
    kds = kernel_descriptors(tmp_path)
    per_rank = {k: v for k, v in kds.items()
                if re.match(r"_ZN2hr(10exchange_k|11exchange2_k|13exchange_ll_k)I", k)}
    group = {k: v for k, v in kds.items() if "_group_k" in k}
    assert len(per_rank) == 3 * 28 and len(group) == 3 * 28, (len(per_rank), len(group))
    length = {k: struct.unpack_from("<H", v, 58)[0] & 0x7F for k, v in kds.items()}
    assert {length[k] for k in per_rank} == {9}
    assert {length[k] for k in group} == {0}
