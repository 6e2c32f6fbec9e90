"""Register and LDS budgets that the mixed-batch split of a CU relies on,
read from the compiler's resource report (CPU: hipcc cross-compiles gfx950).

On a large mixed batch the decode launches run beside the prefill kernel:
the prefill launch asks for enough LDS that one workgroup fits per CU, and
the decode instance built for it holds more than half of a SIMD's 512
registers, so at most one of its waves sits on a SIMD, next to one prefill
wave.  Both hold only if the two register counts stay in these bounds."""
import os
import re
import shutil
import subprocess

import pytest

from ragged_paged_attention_amd import build as pa_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ragged_paged_attention_amd", "csrc")

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="needs hipcc")


def _resources(src):
    """{mangled kernel name: {field: value}} from -Rpass-analysis=kernel-resource-usage."""
    cmd = [pa_build.hipcc()] + pa_build.FLAGS + pa_build.FILE_FLAGS.get(src, []) + [
        "-Rpass-analysis=kernel-resource-usage", "--offload-device-only", "-c", os.path.join(CSRC, src),
        "-o", os.devnull]
    out = subprocess.run(cmd, capture_output=True, text=True, timeout=600).stderr
    res, name = {}, None
    for line in out.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            res[name] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[bytes/[a-z]+\])?: (\d+)", line)
        if m and name:
            res[name][m.group(1).strip()] = int(m.group(2))
    return res


def _regs(r):
    """Registers a wave holds: VGPRs (to a multiple of 4) then AGPRs, in granules of 8."""
    total = (r["VGPRs"] + 3) // 4 * 4 + r.get("AGPRs", 0)
    return (total + 7) // 8 * 8


def test_decode_beside_prefill_register_split():
    dec = _resources("attn_fast.hip")
    pre = _resources("attn_prefill.hip")
    beside = [r for n, r in dec.items() if "decode_kernel" in n and "Li1ELi128ELb1ELb1E" in n]
    prefill = [r for n, r in pre.items() if "prefill_kernel" in n and "Lb1ELi128E" in n]
    assert beside and prefill
    for b in beside:
        assert b.get("VGPRs Spill", 0) == 0 and b.get("ScratchSize", 0) == 0
        assert _regs(b) > 256                    # two of its waves never share a SIMD
        for p in prefill:
            assert _regs(b) + _regs(p) <= 512    # one of each does


def test_bench_kernel_name_fragments_match_built_kernels():
    """bench.py picks each kernel out of rocprofv3 output by a fragment of its
    name; every fragment must match a kernel the sources build (a template
    argument added to a kernel once left a counter summary empty)."""
    filt = shutil.which("c++filt")
    if filt is None:
        pytest.skip("needs c++filt")
    import bench
    names = []
    for src in ("attn_fast.hip", "attn_prefill.hip", "write_kv.hip", "copy_blocks.hip"):
        mangled = list(_resources(src))
        out = subprocess.run([filt], input="\n".join(mangled), capture_output=True, text=True, timeout=60).stdout
        names += [n.replace("(anonymous namespace)::", "") for n in out.splitlines()]
    for kernel, frag in bench.KERNEL_MATCH.items():
        assert any(frag in n for n in names), (kernel, frag)
