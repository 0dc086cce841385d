"""libhr from plain C: the header compiles as strict C99 (CPU), and a C99
program that uses only hr.h and the HIP runtime's C API folds and exchanges
bit-exactly with the oracle (GPU)."""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from message_fp16_all_amd import hr, inputs

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c", "hr_c_client.c")
INC = [os.path.join(ROOT, "include"), "/opt/rocm/include"]


def test_header_is_strict_c99(tmp_path):
    src = tmp_path / "h.c"
    src.write_text('#include "hr.h"\nint main(void) { hr_channel_config c = {0}; (void)c; '
                   'return (int)sizeof(hr_channel_info) > 0 ? 0 : 1; }\n')
    subprocess.run(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
                    "-I", INC[0], "-c", str(src), "-o", str(tmp_path / "h.o")], check=True)


def test_client_compiles_as_c99(tmp_path):
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    *sum([["-I", d] for d in INC], []), "-c", SRC, "-o", str(tmp_path / "c.o")],
                   check=True)


def build_client(tmp_path):
    exe = tmp_path / "hr_c_client"
    libdir = os.path.dirname(hr.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-O2", "-D__HIP_PLATFORM_AMD__",
                    *sum([["-I", d] for d in INC], []), SRC, "-o", str(exe),
                    "-L", libdir, "-lhr", f"-Wl,-rpath,{libdir}",
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    return exe


@pytest.mark.gpu
# (2, 4099) takes the low-latency exchange, (2, 126979) the one-shot
@pytest.mark.parametrize("G,n", [(2, 4096 * 31 + 3), (2, 4099), (8, 393_216)])
def test_c_client_matches_oracle(tmp_path, G, n):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    exe = build_client(tmp_path)
    xs = inputs.contributions(G, n, 1.0, workload=94)
    (tmp_path / "in.bin").write_bytes(np.concatenate(xs).astype(np.uint16).tobytes())
    print(f"c client: G={G} n={n}", flush=True)
    sys.stdout.flush()
    subprocess.run([str(exe), str(G), str(n), str(tmp_path / "in.bin"), str(tmp_path / "out.bin")],
                   check=True, timeout=120)
    got = np.frombuffer((tmp_path / "out.bin").read_bytes(), dtype=np.uint16)
    ref = oracle.fold(xs)
    parts = got.reshape(-1, n)
    # the fold; for two ranks the per-rank exchange's two outputs; for groups
    # of up to eight the group launch's G outputs
    assert parts.shape[0] == 1 + (2 if G == 2 else 0) + (G if 2 <= G <= hr.HR_MAX_WORLD else 0)
    for p in parts:
        assert oracle.same_bits(p, ref).all()
