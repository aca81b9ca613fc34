"""Checks on the gfx950 code object of the built library (no GPU needed).

The kernels are read out of libkda_decode.so itself: its .hip_fatbin section
holds clang offload bundles whose gfx950 entries are the device code objects.  Its
AMDGPU metadata gives each kernel's registers, scratch and spills; its
disassembly shows the instructions the compiler chose.  Checked here:

- every kernel runs without scratch memory and spills no VGPR (the
  admitted launch shapes were chosen so that the state tile stays in VGPRs);
  scalar registers may spill only into lanes of a VGPR (v_writelane /
  v_readlane, no memory access), which a zero private segment confirms;
- every kernel that stores an fp16 state narrows it with v_cvt_pk_f16_f32 or
  v_cvt_f16_f32, which round to nearest even under the default mode, the store the
  fp16 pool is defined with (ROCm/ATOM PR #2945, Summary and Changes), and
  never with the round-toward-zero v_cvt_pkrtz_f16_f32 or a mixed-precision
  fma that rounds straight to fp16 (v_fma_mixlo/hi_f16);
- no kernel contains a packed fp32 instruction (v_pk_fma_f32, v_pk_mul_f32,
  v_pk_add_f32): the build turns that feature off;
- each bundle holds gfx950 device code only.  The section holds one bundle
  per HIP source file (the decode kernels, the prefill kernels); all are read.

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


MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
# one bundle per compiled source file (decode kernels, prefill kernels)
SOURCES_WITH_KERNELS = 2


@pytest.fixture(scope="module")
def code_object(tmp_path_factory):
    """Every offload bundle of the library's .hip_fatbin section (one per
    HIP source file, each aligned), unbundled to its gfx950 code object."""
    if not os.path.exists(LIB):
        pytest.skip("libkda_decode.so is not built")
    d = tmp_path_factory.mktemp("co")
    fatbin = str(d / "fatbin.bin")
    subprocess.run([tool("llvm-objcopy"), "--dump-section=.hip_fatbin=" + fatbin, LIB,
                    str(d / "stripped.so")], check=True)
    data = open(fatbin, "rb").read()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    paths, bundles = [], []
    for i, start in enumerate(starts):
        end = starts[i + 1] if i + 1 < len(starts) else len(data)
        part, co = str(d / ("bundle%d.bin" % i)), str(d / ("gfx950_%d.co" % i))
        with open(part, "wb") as f:
            f.write(data[start:end])
        bundles.append(subprocess.run([tool("clang-offload-bundler"), "--list", "--type=o",
                                       "--input=" + part], check=True, capture_output=True,
                                      text=True).stdout.split())
        subprocess.run([tool("clang-offload-bundler"), "--unbundle", "--type=o", "--input=" + part,
                        "--targets=" + TARGET, "--output=" + co], check=True)
        paths.append(co)
    return {"paths": paths, "bundles": bundles}


@pytest.fixture(scope="module")
def kernels(code_object):
    out = {}
    for path in code_object["paths"]:
        notes = subprocess.run([tool("llvm-readelf"), "--notes", path], check=True,
                               capture_output=True, text=True).stdout
        doc = notes[notes.index("---"):]
        doc = doc[:doc.index("...") + 3] if "..." in doc else doc
        out.update({k[".name"]: k for k in yaml.safe_load(doc)["amdhsa.kernels"]})
    return out


@pytest.fixture(scope="module")
def disassembly(code_object):
    body = {}
    for path in code_object["paths"]:
        text = subprocess.run([tool("llvm-objdump"), "-d", "--no-show-raw-insn", path],
                              check=True, capture_output=True, text=True).stdout
        name = None
        for line in text.splitlines():
            m = re.match(r"^[0-9a-f]+ <(.+)>:$", line)
            if m:
                name = m.group(1)
                body[name] = []
            elif name is not None and line.strip():
                body[name].append(line.split()[0])
    return body


def test_bundles_are_gfx950_device_code_only(code_object):
    assert len(code_object["bundles"]) >= SOURCES_WITH_KERNELS
    for listed in code_object["bundles"]:
        devices = [t for t in listed if not t.startswith("host-")]
        assert devices == [TARGET]


def test_every_source_file_is_checked(kernels):
    # the decode kernels and the prefill kernels come from different bundles
    assert any("kda_decode_tile" in n for n in kernels)
    assert any("kda_rows_kernel" in n for n in kernels)
    assert sum("kda_prefill" in n for n in kernels) == 4


def test_every_kernel_has_no_scratch_and_no_spills(kernels):
    kda = {n: k for n, k in kernels.items() if "kda" in n}
    # decode tiles, chained-row kernels, prefill kernels, copies
    assert len(kda) >= 80
    bad = {n: (k[".private_segment_fixed_size"], k[".vgpr_spill_count"])
           for n, k in kda.items() if k[".private_segment_fixed_size"] or k[".vgpr_spill_count"]}
    assert not bad, bad
    # scalar spills (if any) went to VGPR lanes: no scratch was reserved for them,
    # and only the prefill kernels have any
    sgpr = {n: k[".sgpr_spill_count"] for n, k in kda.items() if k[".sgpr_spill_count"]}
    assert all("kda_prefill" in n for n in sgpr), sgpr
    assert all(v <= 32 for v in sgpr.values()), sgpr


def test_default_single_row_tiles_keep_two_waves_per_simd(kernels):
    # fp32: 2 waves of 32 lanes per 128-column row; fp16: 1 wave of 8 lanes
    # per 64-column row (a SIMD holds 512 VGPRs per lane: two waves need at
    # most 256 each)
    for prefix in ("_ZN3kda15kda_decode_tileIfLi32ELi2ELb0ELb0ELb0EE",
                   "_ZN3kda15kda_decode_tileIDF16_Li8ELi1ELb0ELb0ELb0EE"):
        name = by_prefix(kernels, prefix)
        k = kernels[name]
        assert k[".vgpr_count"] + k.get(".agpr_count", 0) <= 256, (name, k[".vgpr_count"])


def by_prefix(table, prefix):
    """The one kernel symbol that starts with `prefix` (the mangled name up
    to the end of its template arguments; the parameter list may change)."""
    hits = [n for n in table if n.startswith(prefix)]
    assert len(hits) == 1, (prefix, hits)
    return hits[0]


MFMA8 = ("_ZN3kda21kda_rows_mfma8_kernelIfLi0EEE", "_ZN3kda21kda_rows_mfma8_kernelIDF16_Li0EEE")
MFMA8_CONV = ("_ZN3kda21kda_rows_mfma8_kernelIfLi1EEE", "_ZN3kda21kda_rows_mfma8_kernelIDF16_Li1EEE")
MFMA8_CONV_HALF = ("_ZN3kda21kda_rows_mfma8_kernelIfLi2EEE", "_ZN3kda21kda_rows_mfma8_kernelIDF16_Li2EEE")
MFMA4 = ("_ZN3kda20kda_rows_mfma_kernelIfLb0EEE", "_ZN3kda20kda_rows_mfma_kernelIDF16_Lb0EEE")
MFMA4_CONV = ("_ZN3kda20kda_rows_mfma_kernelIfLb1EEE", "_ZN3kda20kda_rows_mfma_kernelIDF16_Lb1EEE")


def test_matrix_block_form_lds_matches_the_launch_description(kernels):
    # the host's LDS figure for the matrix-core block form is the kernel's
    # static LDS, for both pool dtypes and both wave counts
    import kda_gated_delta_decode_amd.binding as B
    for names, nw in ((MFMA8 + MFMA8_CONV_HALF, 8), (MFMA4, 4)):
        want = B.kda_describe_launch(8, 8, 12, "f16", rows_layout=B.KDA_ROWS_MATRIX,
                                     waves_per_tile=nw)["lds_bytes"]
        for prefix in names:
            name = by_prefix(kernels, prefix)
            assert kernels[name][".group_segment_fixed_size"] == want, name
    # with the fused convolution, 8 waves per half: the same arrays with v,
    # the partial sums and their totals for two 64-column halves
    t, k, bh = 8, 128, 64
    conv16 = 4 * (3 * t * (k + 4) + t * 2 * bh + 2 * (8 + 1) * 16 * bh + 2 * t * t + t)
    for prefix in MFMA8_CONV:
        name = by_prefix(kernels, prefix)
        assert kernels[name][".group_segment_fixed_size"] == conv16 <= 160 * 1024, name


def test_fused_sixteen_wave_form_fits_four_waves_per_simd(kernels):
    # 1024 threads: 4 waves per SIMD, at most 128 registers each
    for prefix in MFMA8_CONV:
        name = by_prefix(kernels, prefix)
        k = kernels[name]
        assert k[".max_flat_workgroup_size"] == 1024, name
        assert k[".vgpr_count"] + k.get(".agpr_count", 0) <= 128, (name, k[".vgpr_count"])


def test_matrix_block_form_runs_its_column_sums_on_the_matrix_cores(disassembly):
    # 4 waves: 8 steps of 4 rows x 4 column offsets, 32 fp32 16x16x4 products
    # per wave (with and without the fused convolution); 8 waves: 4 steps, 16
    for prefix in MFMA4 + MFMA4_CONV:
        name = by_prefix(disassembly, prefix)
        assert disassembly[name].count("v_mfma_f32_16x16x4_f32") == 32, name
    for prefix in MFMA8 + MFMA8_CONV + MFMA8_CONV_HALF:
        name = by_prefix(disassembly, prefix)
        assert disassembly[name].count("v_mfma_f32_16x16x4_f32") == 16, name


def test_convolution_in_halves_hands_the_history_over_with_one_counter(disassembly):
    # one relaxed atomic add per workgroup on the pair counter, with no L2
    # write-back or invalidate around it (an agent-scope release would write
    # back the whole L2 of the XCD); the other forms have no atomics
    for prefix in MFMA8_CONV_HALF:
        ops = disassembly[by_prefix(disassembly, prefix)]
        atomics = [op for op in ops if "atomic" in op]
        assert atomics == ["global_atomic_add"], (prefix, atomics)
        assert "buffer_wbl2" not in ops and "buffer_inv" not in ops, prefix
        # issued after the last barrier
        i = ops.index("global_atomic_add")
        barriers = [j for j, op in enumerate(ops) if op == "s_barrier"]
        assert barriers and barriers[-1] < i, prefix
    for prefix in MFMA8 + MFMA8_CONV + MFMA4 + MFMA4_CONV:
        ops = disassembly[by_prefix(disassembly, prefix)]
        assert not any("atomic" in op for op in ops), prefix


def test_pair_counter_result_is_waited_for_only_after_the_snapshots(code_object):
    # no vector-memory wait between the increment and the snapshot stores:
    # the wave that issues it goes on with its solve (the atomic optimizer's
    # rewrite would read the result back at once)
    for prefix in MFMA8_CONV_HALF:
        lines = None
        for path in code_object["paths"]:
            text = subprocess.run([tool("llvm-objdump"), "-d", "--no-show-raw-insn", path],
                                  check=True, capture_output=True, text=True).stdout
            blocks = re.split(r"^[0-9a-f]+ <", text, flags=re.M)
            hit = [b for b in blocks if b.startswith(prefix)]
            if hit:
                lines = [l.split("//")[0].strip() for l in hit[0].splitlines()[1:] if l.strip()]
                break
        assert lines is not None, prefix
        i = next(j for j, l in enumerate(lines) if l.startswith("global_atomic_add"))
        w = next(j for j in range(i, len(lines)) if lines[j].startswith("s_waitcnt") and "vmcnt" in lines[j])
        stores = sum(1 for l in lines[i:w] if l.startswith("global_store_dwordx"))
        assert stores >= 8 * 4, (prefix, stores)   # 8 rows x 4 snapshot pieces per lane


def kernel_lines(code_object, prefix):
    """The disassembled instructions (with operands) of the one kernel whose
    symbol starts with `prefix`."""
    for path in code_object["paths"]:
        text = subprocess.run([tool("llvm-objdump"), "-d", "--no-show-raw-insn", path],
                              check=True, capture_output=True, text=True).stdout
        blocks = re.split(r"^[0-9a-f]+ <", text, flags=re.M)
        hit = [b for b in blocks if b.startswith(prefix)]
        if hit:
            assert len(hit) == 1, prefix
            return [l.split("//")[0].strip() for l in hit[0].splitlines()[1:] if l.strip()]
    raise AssertionError("no kernel " + prefix)


# the fused launches' default kernels: single rows (fp32 over 2 waves, fp16
# over 4), chained rows in 64-column halves and as whole heads
FUSED_DEFAULTS = ("_ZN3kda15kda_decode_tileIfLi32ELi2ELb0ELb1ELb0EE",
                  "_ZN3kda15kda_decode_tileIDF16_Li16ELi4ELb0ELb1ELb0EE") + MFMA8_CONV + MFMA8_CONV_HALF


def test_fused_kernels_issue_the_state_loads_before_any_memory_wait(code_object):
    # the history, row and tap loads of the convolution are issued first and
    # only consumed after the state tile's (nontemporal) loads are in flight:
    # a wait in between would put their round trip in front of the tile's
    for prefix in FUSED_DEFAULTS:
        lines = kernel_lines(code_object, prefix)
        first = next(j for j, l in enumerate(lines) if l.startswith("global_load") and l.endswith(" nt"))
        waits = [l for l in lines[:first] if l.startswith("s_waitcnt") and "vmcnt" in l]
        assert not waits, (prefix, waits)
        assert sum(1 for l in lines[:first] if l.startswith("global_load")) >= 8, prefix


def kernel_descriptor(code_object, name):
    """The 64-byte kernel descriptor (symbol NAME.kd) from whichever code
    object holds it."""
    for path in code_object["paths"]:
        syms = subprocess.run([tool("llvm-readelf"), "-s", "-W", path], check=True,
                              capture_output=True, text=True).stdout
        hit = [l.split() for l in syms.splitlines() if l.split() and l.split()[-1] == name + ".kd"]
        if not hit:
            continue
        value = int(hit[0][1], 16)
        secs = subprocess.run([tool("llvm-readelf"), "-S", "-W", path], check=True,
                              capture_output=True, text=True).stdout
        for line in secs.splitlines():
            f = line.replace("[", " ").replace("]", " ").split()
            if ".rodata" in f:
                i = f.index(".rodata")
                addr, off = int(f[i + 2], 16), int(f[i + 3], 16)
                with open(path, "rb") as fh:
                    fh.seek(off + value - addr)
                    return fh.read(64)
    raise KeyError(name)


def test_leading_arguments_are_preloaded(code_object, kernels):
    # every decode kernel has its leading argument dwords (slot tables, pool,
    # q, k, block count, slot count, packed sizes: 13) preloaded into scalar
    # registers: the descriptor's kernarg_preload field (bytes 58..59, length
    # in bits 0..6)
    decode = [n for n in kernels if n.startswith(("_ZN3kda15kda_decode_tile", "_ZN3kda15kda_rows_kernel",
                                                  "_ZN3kda20kda_rows_mfma_kernel",
                                                  "_ZN3kda21kda_rows_mfma8_kernel"))]
    assert len(decode) >= 50
    for name in decode:
        kd = kernel_descriptor(code_object, name)
        assert int.from_bytes(kd[58:60], "little") & 0x7F >= 13, name


def test_fp16_state_is_narrowed_to_nearest_even(disassembly):
    # every kernel that stores an fp16 state it computed in fp32 (the probes
    # only move bits)
    f16 = {n: ops for n, ops in disassembly.items() if "kda" in n and "DF16_" in n and "probe" not in n}
    assert len(f16) >= 30
    for name, ops in f16.items():
        # packed (decode) or one value at a time (the prefill's final state)
        assert any(op.startswith(("v_cvt_pk_f16_f32", "v_cvt_f16_f32")) for op in ops), name
        for banned in ("v_cvt_pkrtz_f16_f32", "v_fma_mixlo_f16", "v_fma_mixhi_f16",
                       "v_mad_mixlo_f16", "v_mad_mixhi_f16"):
            assert banned not in ops, (name, banned)


def test_no_packed_fp32_instructions(disassembly):
    packed = {"v_pk_fma_f32", "v_pk_mul_f32", "v_pk_add_f32"}
    found = {n: sorted(packed & set(ops)) for n, ops in disassembly.items() if packed & set(ops)}
    assert not found, found
