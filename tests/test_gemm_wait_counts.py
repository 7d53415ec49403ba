"""The fused GEMM's explicit vector-memory wait counts match the loads the
compiled kernels issue.

A wait that keeps the newest N vector-memory operations outstanding is only
right if exactly N operations were issued after the one it waits for.  The
counts in gemm.hip are built from the loads the source issues (the LoRA
seed's 8 DMAs a wave, then the stages of steps 0 and 1: 4 activation DMAs a
step plus, with the in-LDS decode, the codes, the group scale and, with
double quantisation, the 8-bit block code; with the once-per-call
dequantisation 4 weight DMAs instead).  Should the compiler drop a load whose
result one instantiation does not use, a count would be one too large and
the seed would read a stage still in flight.  This compiles gemm.hip for
gfx950 (device code, assembly only; no GPU needed) and checks every GEMM
kernel: the first vector-memory wait after the seed's DMAs keeps exactly the
loads issued after them outstanding.
"""
import os
import re
import shutil
import subprocess

import pytest

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")

KERNEL = re.compile(r"^(_ZN5qlora17qlora_gemm_kernel\w+):[^\n]*\n(.*?)^\.Lfunc_end", re.M | re.S)
LOAD = re.compile(r"^\s*buffer_load_\w+\s")
VMCNT = re.compile(r"s_waitcnt\s.*vmcnt\((\d+)\)")


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    from bit_nf4_quantized_06_amd import build as B
    out = tmp_path_factory.mktemp("asm") / "gemm.s"
    cmd = [HIPCC] + B.hipcc_flags() + ["--cuda-device-only", "-S", "-o", str(out),
                                       os.path.join(B.CSRC, "gemm.hip")]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    return out.read_text()


def test_every_gemm_kernel_waits_for_exactly_its_seed_loads(gemm_asm):
    kernels = KERNEL.findall(gemm_asm)
    # <backward, dropout, double quantisation, fp16, once-per-call dequantisation>:
    # 3 weight formats x 2 compute types x (forward, backward, backward with
    # dropout), the dequantised-weight path in either compute type
    assert len(kernels) == 18, [k for k, _ in kernels]
    seen = set()
    for name, body in kernels:
        lines = body.splitlines()
        first = next(i for i, l in enumerate(lines) if LOAD.match(l) and l.rstrip().endswith(" lds"))
        wait = next(i for i in range(first, len(lines)) if VMCNT.search(lines[i]))
        kept = int(VMCNT.search(lines[wait]).group(1))
        issued = sum(1 for l in lines[first:wait] if LOAD.match(l))
        assert issued == 8 + kept, f"{name}: {issued} loads before a wait keeping {kept}"
        seen.add(kept)
    # the three prologue shapes: dequantised weight (3 x 4 DMAs), in-LDS decode
    # with (2 x 7) and without (2 x 6) double quantisation
    assert seen == {12, 14}, seen
