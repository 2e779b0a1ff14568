"""Checks on the gfx950 assembly of the kernels (CPU only: hipcc cross-compiles).

The prefill kernel issues its global -> LDS copies through inline assembly that
writes m0, a register the compiler reserves; that is sound only while nothing
else in the kernel relies on m0, and the LDS-DMA load needs one wait state
after the m0 write.  Both are checked on the generated code."""
import os
import re
import shutil
import subprocess

import pytest

from paged_kv_gqa_mapping_amd import build as B

HIPCC = next((c for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc"))
              if c and os.path.exists(c)), None)


def _device_asm(src: str, tmp_path) -> str:
    out = tmp_path / "k.s"
    cmd = [HIPCC, *B.FLAGS, "-I", B.CSRC, "--cuda-device-only", "-S", "-x", "hip",
           os.path.join(B.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    return out.read_text()


@pytest.mark.skipif(HIPCC is None, reason="hipcc not found")
def test_prefill_m0_is_only_written_by_the_copy_sequence(tmp_path):
    lines = [ln.split(";")[0].strip() for ln in _device_asm("prefill_mfma.hip", tmp_path).splitlines()]
    lines = [ln for ln in lines if ln]
    copies = 0
    for i, ln in enumerate(lines):
        if not re.search(r"\bm0\b", ln):
            continue
        assert re.fullmatch(r"s_mov_b32 m0, s\d+", ln), f"unexpected m0 use: {ln}"
        assert lines[i + 1] == "s_nop 0", f"no wait state after {ln}: {lines[i + 1]}"
        assert lines[i + 2].startswith("global_load_lds_dwordx4 "), f"{ln} not followed by the copy: {lines[i + 2]}"
        copies += 1
    assert copies > 0
    # the copies are the only LDS-DMA loads, so each one is preceded by its m0 write
    assert sum(ln.startswith("global_load_lds") for ln in lines) == copies


@pytest.mark.skipif(HIPCC is None, reason="hipcc not found")
def test_prefill_kernels_do_not_spill(tmp_path):
    text = _device_asm("prefill_mfma.hip", tmp_path)
    sizes = [int(x) for x in re.findall(r"\.private_segment_fixed_size:\s+(\d+)", text)]
    assert sizes and all(x == 0 for x in sizes), sizes


@pytest.mark.skipif(HIPCC is None, reason="hipcc not found")
def test_bf16_decode_kernels_do_not_spill(tmp_path):
    # the bf16 decode split pass holds up to three steps of K/V rows in registers
    # (256 VGPRs plus accumulation registers for four query heads per KV head):
    # any scratch use there would put memory round trips in the stream
    text = _device_asm("row_attn.hip", tmp_path)
    sizes = {}
    name = None
    for ln in text.splitlines():
        m = re.match(r"\s*\.amdhsa_kernel\s+(\S+)", ln)
        if m:
            name = m.group(1)
        m = re.match(r"\s*\.amdhsa_private_segment_fixed_size\s+(\d+)", ln)
        if m and name:
            sizes[name] = int(m.group(1))
    bf16 = {k: v for k, v in sizes.items()
            if k.startswith("_ZN3pkv15row_attn_kernelILb1E") or k.startswith("_ZN3pkv20decode_reduce_kernelILb1E")}
    assert len(bf16) >= 10, sorted(sizes)
    assert all(v == 0 for v in bf16.values()), {k: v for k, v in bf16.items() if v}
