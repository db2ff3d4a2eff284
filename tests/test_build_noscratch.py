"""The built library's E4M3 x E4M3 GEMM kernels keep all their state in
registers: no kernel has a private (scratch) segment.  A spill inside a K loop
is a reload from memory, and the compiler's wait for it also waits for the
asynchronous operand copies in flight, which serialises the pipeline (a
spill of two values once cost 15 % on the row-scaled 4096^3 GEMM).

Reads the code objects that hipcc embedded in libdg.so (the .hip_fatbin
section, one offload bundle per translation unit) with the ROCm LLVM tools;
runs on the CPU and is skipped when the library or the tools are missing."""
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "moe_grouped_gemm_block_amd", "libdg.so")
TOOLS = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
# operand-format suffixes of the mixed / E5M2 kernels; their row-scaled
# 128 x 512 and 256 x 256 variants need a few registers more than there are
OTHER_FORMATS = ("_a4b5", "_a5b4", "_a5b5")


def kernel_scratch():
    """{kernel symbol: private segment bytes} over every gfx950 code object."""
    for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf"):
        if not os.path.exists(os.path.join(TOOLS, t)):
            pytest.skip(f"{t} not found")
    if not os.path.exists(LIB):
        pytest.skip("libdg.so is not built")
    out = {}
    with tempfile.TemporaryDirectory() as tmp:
        fat = os.path.join(tmp, "fatbin")
        subprocess.run([os.path.join(TOOLS, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", LIB,
                        os.path.join(tmp, "lib.copy")], check=True, capture_output=True)
        data = open(fat, "rb").read()
        starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
        assert starts, "no offload bundle in .hip_fatbin"
        for i, s in enumerate(starts):
            part = os.path.join(tmp, f"b{i}")
            open(part, "wb").write(data[s:starts[i + 1] if i + 1 < len(starts) else len(data)])
            co = os.path.join(tmp, f"co{i}")
            subprocess.run([os.path.join(TOOLS, "clang-offload-bundler"), "--unbundle", "--type=o",
                            f"--input={part}", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"],
                           check=True, capture_output=True)
            notes = subprocess.run([os.path.join(TOOLS, "llvm-readelf"), "--notes", co], check=True,
                                   capture_output=True, text=True).stdout
            name = None
            for line in notes.splitlines():
                m = re.match(r"\s+\.name:\s+(\S+)", line)
                if m:
                    name = m.group(1)
                m = re.match(r"\s+\.private_segment_fixed_size:\s+(\d+)", line)
                if m and name is not None:
                    out[name] = int(m.group(1))
                    name = None
    return out


def test_e4m3_gemm_kernels_do_not_spill():
    sizes = kernel_scratch()
    gemm = {k: v for k, v in sizes.items()
            if re.search(r"dg_(gemm|skinny|segments)_", k) and not any(f in k for f in OTHER_FORMATS)}
    # tiled shapes (with and without row scales), few-rows and packed-segment kernels
    for shape in ("sb256", "128x512", "128x256", "128x256w8", "128x128w4", "128x64w2", "skinny_m64",
                  "segments_n48"):
        assert any(shape in k for k in gemm), f"no {shape} kernel found"
    spilled = {k: v for k, v in gemm.items() if v != 0}
    assert not spilled, f"kernels with scratch: {spilled}"
