"""Properties of the compiled gfx950 device code, checked on the CPU (hipcc
cross-compiles each source to assembly here).

- No flat memory instructions anywhere.  Every kernel addresses device
  memory through buffer resources or global pointers; a flat access (what
  the compiler emits when it cannot prove a pointer global) also counts on
  the LDS counter, so the next LDS wait would drain every load in flight.
  That has cost a verify call 0.2 us once already.
- No scratch (register spills) in any kernel, except the two bf16 verify
  chunk forms at 512 head dims, which hold both 128-key halves' K operands
  in registers and spill 20-24 bytes a lane; no benchmarked shape uses them.
"""
from __future__ import annotations

import concurrent.futures as cf
import importlib.util
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sliding_window_ring_amd", "csrc")

SCRATCH_ALLOWED = {
    "_ZN3swr12chunk_kernelILi512ELi2ELb0ELi1ELb0EEEvNS_10AttnParamsE",  # verify, bf16, D=512, 32 rows
    "_ZN3swr12chunk_kernelILi512ELi1ELb0ELi1ELb0EEEvNS_10AttnParamsE",  # verify, bf16, D=512, 16 rows
}


def _build_module():
    spec = importlib.util.spec_from_file_location("_swr_build", os.path.join(ROOT, "sliding_window_ring_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    b = _build_module()
    if not os.path.exists(b.HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm")
    srcs = [s for s in b.SOURCES if s.endswith(".hip")]

    def compile_one(src):
        dst = os.path.join(out, src + ".s")
        cmd = [b.HIPCC, *[f for f in b.CFLAGS if f != "-fPIC"], "-x", "hip", "--offload-device-only", "-S",
               os.path.join(CSRC, src), "-o", dst]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        assert r.returncode == 0, r.stdout
        with open(dst) as f:
            return src, f.read()

    with cf.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        return dict(ex.map(compile_one, srcs))


def kernel_bodies(text):
    """(symbol, instructions) of every kernel in one assembly file: from the
    kernel's label to the end of its function (past every exit)."""
    out = {}
    for name in re.findall(r"\.amdhsa_kernel (\S+)", text):
        m = re.search(r"^" + re.escape(name) + r":.*?$(.*?)^\.Lfunc_end\d+:", text, re.M | re.S)
        assert m, f"no code found for {name}"
        out[name] = m.group(1)
    return out


def test_every_kernel_source_has_kernels(device_asm):
    for src, text in device_asm.items():
        with open(os.path.join(CSRC, src)) as f:
            defines = "__global__" in f.read()
        assert bool(kernel_bodies(text)) == defines, f"{src}: kernels in the assembly do not match the source"


def test_no_flat_memory_instructions(device_asm):
    bad = []
    for src, text in device_asm.items():
        for name, body in kernel_bodies(text).items():
            n = len(re.findall(r"^\s*flat_\w+", body, re.M))
            if n:
                bad.append(f"{src}: {name}: {n}")
    assert not bad, "flat memory instructions:\n" + "\n".join(bad)


def test_scratch_only_where_stated(device_asm):
    seen = {}
    for text in device_asm.values():
        for m in re.finditer(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", text, re.S):
            size = re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", m.group(2))
            seen[m.group(1)] = int(size.group(1))
    assert seen, "no kernel descriptors found"
    spilled = {k for k, v in seen.items() if v > 0}
    assert spilled <= SCRATCH_ALLOWED, f"kernels with scratch: {sorted(spilled - SCRATCH_ALLOWED)}"
