"""Guard for the inline-assembly global->LDS copies of the ping-pong kernel.

The copies set M0 (the LDS destination) right before each
global_load_lds_dwordx4, or before a pair of them that differ only in the
immediate offset (-4096, then 0: the offset moves the global and the LDS
address alike), from inline assembly.  That is only sound while no
compiler-generated instruction in the kernel uses M0.  This test compiles the
library to gfx950 assembly (no GPU needed) and checks, in every kernel that
issues such copies, that each write of M0 is immediately followed by a copy or
such a pair, that every copy follows its M0 write that way, and that no other
instruction that reads M0 implicitly appears.
"""
import os
import re
import subprocess

import pytest

from tiled_online_softmax_causal_amd import build as fa_build

# instructions that read M0 implicitly on gfx9 (besides the LDS copies themselves)
M0_READERS = re.compile(r"\b(s_sendmsg|s_movrel|v_movrel|ds_gws|v_interp|s_set_gpr_idx|ds_.*_addtid|"
                        r"buffer_load_\w+\s.*\blds\b|global_load_lds_(?!dwordx4))")


M0_WRITE = r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)$"


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("isa") / "fa.s"
    cmd = [fa_build.hipcc(), "--offload-arch=gfx950", "--cuda-device-only", "-S", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fno-honor-nans",
           "-I", os.path.join(fa_build.ROOT, "include"), "-I", fa_build.CSRC,
           os.path.join(fa_build.CSRC, "fa_api.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


def _kernels(asm: str):
    """(name, instruction lines) for every kernel body in the assembly.

    A body runs from the kernel's label to its .Lfunc_end label, so kernels with
    several exits (s_endpgm) are read whole."""
    out, name, body = [], None, []
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            name, body = m.group(1), []
            continue
        if name is None:
            continue
        if line.startswith(".Lfunc_end"):
            out.append((name, body))
            name = None
            continue
        text = line.split(";")[0].strip()
        if text and not text.startswith("."):
            body.append(text)
    return out


def test_m0_is_only_the_lds_copy_destination(device_asm):
    kernels = _kernels(device_asm)
    copying = [(n, b) for n, b in kernels if any(i.startswith("global_load_lds_dwordx4") for i in b)]
    assert copying, "no kernel issues global->LDS copies"
    assert any("attn_fwd_pingpong" in n for n, _ in copying)
    for name, body in copying:
        for k, ins in enumerate(body):
            assert not M0_READERS.search(ins), f"{name}: unexpected M0 reader: {ins}"
            if re.search(r"\bm0\b", ins):
                # the LDS address, from whatever scalar register holds it
                assert re.match(M0_WRITE, ins), f"{name}: M0 written by: {ins}"
                assert body[k + 1].startswith("global_load_lds_dwordx4"), f"{name}: M0 write not followed by a copy"
            if ins.startswith("global_load_lds_dwordx4"):
                if re.match(M0_WRITE, body[k - 1]):
                    continue
                # the second copy of a pair: same operands, immediate 0, after the
                # first at -4096, which follows the M0 write
                first = body[k - 1]
                assert first.startswith("global_load_lds_dwordx4") and first.endswith("offset:-4096") \
                    and re.match(M0_WRITE, body[k - 2]), f"{name}: copy without its M0 write: {ins}"
                assert first[:-len(" offset:-4096")] == ins, f"{name}: pair with different operands: {first} / {ins}"


def test_copy_base_is_not_sign_extended(device_asm):
    """The copies take a wave-uniform 64-bit tile address in SGPRs, rebuilt from
    two readfirstlane results.  readfirstlane yields a signed 32-bit value: widened
    without a cast to unsigned, the low word is sign-extended (s_bfe_i64) and an
    address whose bit 31 is set gets an all-ones high word, which faults.  No
    kernel that issues copies may sign-extend a 64-bit scalar."""
    for name, body in _kernels(device_asm):
        if any(i.startswith("global_load_lds_dwordx4") for i in body):
            bad = [i for i in body if i.startswith("s_bfe_i64") or i.startswith("s_sext_i32")]
            assert not bad, f"{name}: sign extension of a scalar: {bad[:3]}"
