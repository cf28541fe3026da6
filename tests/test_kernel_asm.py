"""Properties of the generated gfx950 code that the kernel source relies on.

The direct K/V loads set M0 (the LDS base of an LDS-destination load) from
inline assembly, saving it once per run of loads instead of once per load.
That is only sound while no compiler-generated instruction of these kernels
reads or writes M0, so the assembly is checked for exactly that.  The
kernels are also meant to run without scratch memory (no register spills).
Compiles the kernel source with the library's own flags; no GPU needed.
"""

import os
import re
import subprocess

import pytest

from flash_attention_head_amd import build as B

KERNELS = ("attn_tile_kernel_d256_pers", "attn_tile_kernel_d64", "attn_tile_kernel_d80", "attn_tile_kernel_d128", "attn_tile_kernel_d192", "attn_tile_kernel_dk192_dv256", "attn_tile_kernel_d256",
           "attn_tile_kernel_d512", "attn_tile_kernel_d256_q4", "attn_q4_decode_kernel",
           "combine_kernel", "combine_few_kernel")

# the sources that hold kernels
KERNEL_SOURCES = [s for s in B.SOURCES if os.path.basename(s) in ("attn_kernels.hip", "attn_q4_decode.hip")]


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    assert len(KERNEL_SOURCES) == 2, B.SOURCES
    d = tmp_path_factory.mktemp("asm")
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC", "-fvisibility=hidden")]
    text = []
    for src in KERNEL_SOURCES:
        out = str(d / (os.path.basename(src) + ".s"))
        r = subprocess.run([B.HIPCC, *flags, "--cuda-device-only", "-S", src, "-o", out], capture_output=True,
                           text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        text.append(open(out).read())
    return "\n".join(text)


def _functions(text):
    """name -> body lines of every kernel in the assembly listing."""
    funcs = {}
    for m in re.finditer(r"^(_Z\S+):", text, re.M):
        name = m.group(1)
        if not any(k in name for k in KERNELS):
            continue
        end = text.index("s_endpgm", m.end())
        funcs[name] = text[m.end():end].splitlines()
    return funcs


def test_every_kernel_instance_is_present(asm):
    names = list(_functions(asm))
    for k in KERNELS:
        assert sum(k in n for n in names) >= 2, (k, names)  # fp16 and bf16 instances


def test_m0_is_touched_only_by_the_inline_assembly(asm):
    for name, lines in _functions(asm).items():
        inside = False
        for ln in lines:
            if ";;#ASMSTART" in ln:
                inside = True
            elif ";;#ASMEND" in ln:
                inside = False
            else:
                code = ln.split(";")[0]
                assert inside or not re.search(r"\bm0\b", code), (name, ln)


def _metadata(text):
    """kernel name -> its code-object metadata fields (name: value strings)."""
    kernels = {}
    for block in re.split(r"\n\s+- \.", text):
        m = re.search(r"\.name:\s+(\S+)", block)
        if m and any(k in m.group(1) for k in KERNELS):
            kernels[m.group(1)] = dict(re.findall(r"\.(\w+):\s+(\S+)", block))
    return kernels


# The 4-bit instances (their loaders' register sets live beside the compute
# state) move a few vector registers into the register file's accumulation
# half (v0..v255 are the registers ordinary vector instructions address; the
# spills go to a256 and up): no memory traffic, a register-to-register copy
# each.
SPILL_TO_REGISTERS_ONLY = ("attn_tile_kernel_d256_q4",)


def test_no_scratch_memory(asm):
    """No kernel touches scratch memory or spills vector registers.  Only the
    wrapped-ring and bias instances (a template flag true, "Lb1") may park
    scalar registers in vector-register lanes, and the instance named above
    vector registers in accumulation registers: neither is memory traffic.
    The persistent instance keeps every scalar in a scalar register: its
    direct loads form their LDS address from one base per buffer."""
    meta = _metadata(asm)
    assert len(meta) >= 26, sorted(meta)
    for name, f in meta.items():
        assert int(f["private_segment_fixed_size"]) == 0, (name, f)
        if not any(k in name for k in SPILL_TO_REGISTERS_ONLY):
            assert int(f["vgpr_spill_count"]) == 0, (name, f)
        else:
            assert int(f["vgpr_spill_count"]) <= 8, (name, f)
        if "attn_tile_kernel" in name and "Lb1" not in name:
            assert int(f["sgpr_spill_count"]) == 0, (name, f)
