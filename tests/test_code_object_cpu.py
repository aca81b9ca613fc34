"""Checks on the gfx950 code object of the built library (no GPU needed).

The kernels are read out of libkda_decode.so itself: its .hip_fatbin section
is a clang offload bundle whose gfx950 entry is the device code object.  Its
AMDGPU metadata gives each kernel's registers, scratch and spills; its
disassembly shows the instructions the compiler chose.  Checked here:

- every kernel runs without scratch memory and spills no register (the
  admitted launch shapes were chosen so that the state tile stays in VGPRs);
- every kernel that stores an fp16 state narrows it with v_cvt_pk_f16_f32,
  which rounds to nearest even under the default rounding mode, the store the
  fp16 pool is defined with (ROCm/ATOM PR #2945, Summary and Changes), and
  never with the round-toward-zero v_cvt_pkrtz_f16_f32 or a mixed-precision
  fma that rounds straight to fp16 (v_fma_mixlo/hi_f16);
- no kernel contains a packed fp32 instruction (v_pk_fma_f32, v_pk_mul_f32,
  v_pk_add_f32): the build turns that feature off;
- the bundle holds gfx950 device code only.

Needs the built library and ROCm's LLVM tools (llvm-objcopy,
clang-offload-bundler, llvm-readelf, llvm-objdump); skips if either is absent.
"""
import os
import re
import shutil
import subprocess

import pytest
import yaml

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "kda_gated_delta_decode_amd", "libkda_decode.so")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"


def tool(name):
    path = os.path.join(LLVM, name)
    if not os.path.exists(path):
        path = shutil.which(name)
    if not path:
        pytest.skip("ROCm LLVM tool %s not found" % name)
    return path


@pytest.fixture(scope="module")
def code_object(tmp_path_factory):
    if not os.path.exists(LIB):
        pytest.skip("libkda_decode.so is not built")
    d = tmp_path_factory.mktemp("co")
    fatbin, co = str(d / "fatbin.bin"), str(d / "gfx950.co")
    subprocess.run([tool("llvm-objcopy"), "--dump-section=.hip_fatbin=" + fatbin, LIB,
                    str(d / "stripped.so")], check=True)
    listed = subprocess.run([tool("clang-offload-bundler"), "--list", "--type=o", "--input=" + fatbin],
                            check=True, capture_output=True, text=True).stdout.split()
    subprocess.run([tool("clang-offload-bundler"), "--unbundle", "--type=o", "--input=" + fatbin,
                    "--targets=" + TARGET, "--output=" + co], check=True)
    return {"path": co, "bundle": listed}


@pytest.fixture(scope="module")
def kernels(code_object):
    notes = subprocess.run([tool("llvm-readelf"), "--notes", code_object["path"]], check=True,
                           capture_output=True, text=True).stdout
    doc = notes[notes.index("---"):]
    doc = doc[:doc.index("...") + 3] if "..." in doc else doc
    meta = yaml.safe_load(doc)
    return {k[".name"]: k for k in meta["amdhsa.kernels"]}


@pytest.fixture(scope="module")
def disassembly(code_object):
    text = subprocess.run([tool("llvm-objdump"), "-d", "--no-show-raw-insn", code_object["path"]],
                          check=True, capture_output=True, text=True).stdout
    body, name = {}, None
    for line in text.splitlines():
        m = re.match(r"^[0-9a-f]+ <(.+)>:$", line)
        if m:
            name = m.group(1)
            body[name] = []
        elif name is not None and line.strip():
            body[name].append(line.split()[0])
    return body


def test_bundle_is_gfx950_device_code_only(code_object):
    devices = [t for t in code_object["bundle"] if not t.startswith("host-")]
    assert devices == [TARGET]


def test_every_kernel_has_no_scratch_and_no_spills(kernels):
    kda = {n: k for n, k in kernels.items() if "kda" in n}
    # decode tiles, chained-row kernels, prefill kernels, copies
    assert len(kda) >= 80
    bad = {n: (k[".private_segment_fixed_size"], k[".vgpr_spill_count"], k[".sgpr_spill_count"])
           for n, k in kda.items()
           if k[".private_segment_fixed_size"] or k[".vgpr_spill_count"] or k[".sgpr_spill_count"]}
    assert not bad, bad


def test_default_single_row_tiles_keep_two_waves_per_simd(kernels):
    # fp32: 2 waves of 32 lanes per 128-column row; fp16: 4 waves of 16 lanes
    # (a SIMD holds 512 VGPRs per lane: two waves need at most 256 each)
    for name in ("_ZN3kda15kda_decode_tileIfLi32ELi2ELb0ELb0ELb0EEEvNS_4ArgsE",
                 "_ZN3kda15kda_decode_tileIDF16_Li16ELi4ELb0ELb0ELb0EEEvNS_4ArgsE"):
        k = kernels[name]
        assert k[".vgpr_count"] + k.get(".agpr_count", 0) <= 256, (name, k[".vgpr_count"])


def test_fp16_state_is_narrowed_to_nearest_even(disassembly):
    f16 = {n: ops for n, ops in disassembly.items() if "kda" in n and "DF16_" in n}
    assert len(f16) >= 30
    for name, ops in f16.items():
        assert "v_cvt_pk_f16_f32" in ops, name
        for banned in ("v_cvt_pkrtz_f16_f32", "v_fma_mixlo_f16", "v_fma_mixhi_f16",
                       "v_mad_mixlo_f16", "v_mad_mixhi_f16"):
            assert banned not in ops, (name, banned)


def test_no_packed_fp32_instructions(disassembly):
    packed = {"v_pk_fma_f32", "v_pk_mul_f32", "v_pk_add_f32"}
    found = {n: sorted(packed & set(ops)) for n, ops in disassembly.items() if packed & set(ops)}
    assert not found, found
