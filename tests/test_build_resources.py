"""Resource checks on the built library's gfx950 code objects (no GPU needed).

Every kernel must run without scratch memory: a non-zero private segment
means registers spilled to memory inside the kernel, which costs bandwidth and
latency on the hot path.  The kernel descriptors' metadata is read from the
HIP fat binary embedded in libosattn.so with the ROCm LLVM tools."""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(os.path.dirname(HERE), "online_softmax_attention_amd", "libosattn.so")
LLVM = "/opt/rocm/llvm/bin"
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def kernel_private_segments(lib: str, tmp: str) -> dict:
    """{kernel symbol: private segment bytes per lane} for the gfx950 code."""
    sec = os.path.join(tmp, "fatbin.bin")
    # An explicit output file: without one objcopy rewrites its input in place.
    subprocess.run(["objcopy", "--dump-section", ".hip_fatbin=" + sec, lib,
                    os.path.join(tmp, "lib_copy.so")], check=True, capture_output=True)
    data = open(sec, "rb").read()
    starts = [m.start() for m in re.finditer(re.escape(BUNDLE_MAGIC), data)]
    out = {}
    for i, start in enumerate(starts):  # one bundle per translation unit
        end = starts[i + 1] if i + 1 < len(starts) else len(data)
        chunk = os.path.join(tmp, "bundle%d.bin" % i)
        with open(chunk, "wb") as f:
            f.write(data[start:end])
        obj = os.path.join(tmp, "bundle%d.o" % i)
        subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--type=o", "--input=" + chunk,
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", "--output=" + obj, "--unbundle"],
                       check=True, capture_output=True)
        notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", obj], check=True,
                               capture_output=True, text=True).stdout
        # Each kernel's metadata map lists its keys in order: the private
        # segment size comes before the descriptor symbol.
        for size, sym in re.findall(r"\.private_segment_fixed_size:\s+(\d+).*?\.symbol:\s+(\S+)",
                                    notes, re.S):
            out[sym[:-3] if sym.endswith(".kd") else sym] = int(size)
    return out


@pytest.mark.skipif(not os.path.exists(LIB), reason="libosattn.so is not built")
@pytest.mark.skipif(shutil.which("objcopy") is None or not os.path.exists(LLVM),
                    reason="objcopy or the ROCm LLVM tools are missing")
def test_no_kernel_uses_scratch(tmp_path):
    sizes = kernel_private_segments(LIB, str(tmp_path))
    assert len(sizes) > 50, "expected the library's kernels, found %d" % len(sizes)
    spilled = {k: v for k, v in sizes.items() if v}
    assert not spilled, "kernels with scratch (bytes per lane): %s" % spilled
