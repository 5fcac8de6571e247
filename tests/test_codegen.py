"""Checks on the gfx950 machine code of the built library (no GPU needed).

The global->LDS tile copies are inline assembly, and the compiler's hazard
checks do not look inside inline assembly.  The CDNA ISA asks for one wait
state between a scalar write of M0 and an LDS-bound buffer load, and five
between a vector instruction that writes an SGPR (for instance
v_readlane_b32 restoring a spilled descriptor) and a buffer load that reads
it.  Every such copy must therefore be issued right after `s_nop 4` or a
longer one.  This test disassembles every gfx950 code object in
libfat5attn.so and checks that, and that no kernel spills to scratch (a
spill would also mean the kernel runs far below its design occupancy): no
VGPR spill and no private segment.  SGPRs the compiler parks in spare VGPR
lanes (v_writelane / v_readlane, no memory) are allowed, up to a few per
kernel."""
import os
import re
import shutil
import subprocess

import pytest

from attention_t5_relative_amd import _lib

LLVM = "/opt/rocm/llvm/bin"
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"


def _tool(name):
    path = os.path.join(LLVM, name)
    if not os.path.exists(path):
        pytest.skip(f"{path} not present")
    return path


@pytest.fixture(scope="module")
def code_objects(tmp_path_factory):
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("library not built")
    objcopy, bundler = _tool("llvm-objcopy"), _tool("clang-offload-bundler")
    tmp = tmp_path_factory.mktemp("co")
    fatbin = tmp / "fatbin"
    subprocess.run([objcopy, "--dump-section", f".hip_fatbin={fatbin}", _lib.LIB_PATH],
                   check=True)
    blob = fatbin.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(BUNDLE_MAGIC), blob)]
    assert starts, "no offload bundle in .hip_fatbin"
    objs = []
    for i, s in enumerate(starts):
        end = starts[i + 1] if i + 1 < len(starts) else len(blob)
        part = tmp / f"bundle{i}"
        part.write_bytes(blob[s:end])
        out = tmp / f"gfx950_{i}.o"
        subprocess.run([bundler, "--unbundle", "--type=o", f"--input={part}",
                        f"--targets={TARGET}", f"--output={out}"], check=True)
        objs.append(out)
    return objs


def _disasm(obj):
    return subprocess.run([_tool("llvm-objdump"), "-d", "--mcpu=gfx950", str(obj)],
                          capture_output=True, text=True, check=True).stdout


def test_every_lds_copy_follows_five_wait_states(code_objects):
    total = 0
    bad = []
    for obj in code_objects:
        prev = ""
        func = ""
        for line in _disasm(obj).splitlines():
            m = re.match(r"^[0-9a-f]+ <(\S+)>:$", line)
            if m:
                func, prev = m.group(1), ""
                continue
            ins = line.split("//")[0].strip()
            if not ins:
                continue
            if ins.startswith("buffer_load") and ins.endswith(" lds"):
                total += 1
                nop = re.match(r"s_nop (\d+)$", prev)
                if not nop or int(nop.group(1)) < 4:
                    bad.append(f"{func}: '{prev}' before '{ins}'")
            prev = ins
    assert total > 0, "expected LDS-bound copies in the attention kernels"
    assert not bad, "\n".join(bad[:10])


def test_no_kernel_uses_scratch(code_objects):
    readelf = _tool("llvm-readelf")
    kernels = 0
    for obj in code_objects:
        notes = subprocess.run([readelf, "--notes", str(obj)], capture_output=True, text=True,
                               check=True).stdout
        vspills = re.findall(r"\.vgpr_spill_count:\s+(\d+)", notes)
        sspills = re.findall(r"\.sgpr_spill_count:\s+(\d+)", notes)
        kernels += len(vspills)
        if not vspills:   # a code object holding device data only (the static scratch)
            continue
        assert all(int(n) == 0 for n in vspills), f"{obj.name}: VGPR spills {set(vspills)}"
        # SGPR spills go to VGPR lanes while the private segment stays empty
        assert all(int(n) <= 8 for n in sspills), f"{obj.name}: SGPR spills {set(sspills)}"
        priv = re.findall(r"\.private_segment_fixed_size:\s+(\d+)", notes)
        assert all(int(n) == 0 for n in priv), f"{obj.name}: private segment {set(priv)}"
    assert kernels > 0, "no kernel metadata found"
