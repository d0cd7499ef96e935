"""Register spills of the built gfx950 kernels, read from the code-object metadata of the objects
that build() leaves in decode_attention_06_amd/_build (no GPU needed).  A spill in a hot kernel
turns into scratch-memory traffic on every tile -- a small source edit once added 42 VGPR spills
to the 128K MQA variant and 16 % more HBM reads -- so the variants the workloads run are held at
zero here:
  * every 16-head partition kernel and every combine kernel: 0 VGPR spills;
  * the wide-group kernel with a per-tensor scale (the MQA workloads) or none (f16 / bf16 KV): 0;
  * the wide-group kernel with per-token scales: at most 8 (a known cost at three waves per SIMD;
    no benchmark workload is wide with per-token scales).
Skipped when the objects or the LLVM tools are not there."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "decode_attention_06_amd", "_build")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"


def kernel_spills(obj: str) -> dict:
    """{mangled kernel name: VGPR spill count} of the gfx950 code object inside a HIP object."""
    tools = [os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf")]
    if not all(os.path.exists(t) for t in tools) or not os.path.exists(obj):
        pytest.skip("built objects or LLVM tools not available")
    objcopy, bundler, readelf = tools
    with tempfile.TemporaryDirectory() as d:
        fat, co = os.path.join(d, "fatbin.bin"), os.path.join(d, "k.co")
        subprocess.run([objcopy, f"--dump-section=.hip_fatbin={fat}", obj], check=True, capture_output=True)
        subprocess.run([bundler, "--type=o", f"--targets={TARGET}", f"--input={fat}", f"--output={co}",
                        "--unbundle"], check=True, capture_output=True)
        notes = subprocess.run([readelf, "--notes", co], check=True, capture_output=True, text=True).stdout
    out, name = {}, None
    for line in notes.splitlines():
        m = re.match(r"\s*-?\s*\.name:\s+(_Z\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.match(r"\s*\.vgpr_spill_count:\s+(\d+)", line)
        if m and name:
            out[name] = int(m.group(1))
            name = None
    return out


def test_partition_and_combine_kernels_do_not_spill():
    sp = kernel_spills(os.path.join(BUILD, "fd_kernels.hip.o"))
    part = {k: v for k, v in sp.items() if "partition_kernel" in k}
    comb = {k: v for k, v in sp.items() if "combine_kernel" in k}
    assert part and comb
    assert all(v == 0 for v in part.values()), {k: v for k, v in part.items() if v}
    assert all(v == 0 for v in comb.values()), {k: v for k, v in comb.items() if v}


def test_wide_kernel_spills():
    sp = kernel_spills(os.path.join(BUILD, "fd_wide.hip.o"))
    assert sp
    # template arguments <KVT, WPG, NSLOT, QT, SCALE, PAGED, B16>: SCALE 0 = none, 1 = per tensor,
    # 2 = per token; KVT 1 / 2 = f16 / bf16
    kvts = set()
    for k, v in sp.items():
        m = re.search(r"wide_partition_kernelILi(\d)ELi(\d)ELi(\d)ELi(\d)ELi(\d)E", k)
        assert m, k
        kvts.add(int(m.group(1)))
        scale = int(m.group(5))
        assert v <= (8 if scale == 2 else 0), (k, v)
    assert kvts == {1, 2, 3, 4}, kvts


def test_direct_kernel_spills():
    # the 32-column kernel holds two register tiles (66 VGPRs) and the accumulator (64) across the
    # loop (q's E4M3 terms live in LDS): a reload from scratch inside the loop would also wait for
    # the next tile's loads (scratch shares their counter), so none is allowed
    sp = kernel_spills(os.path.join(BUILD, "fd_direct.hip.o"))
    assert sp
    assert all(v == 0 for v in sp.values()), {k: v for k, v in sp.items() if v}

