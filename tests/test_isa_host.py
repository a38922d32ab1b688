"""Checks on the gfx950 assembly of the attention kernels (built here from source, no GPU needed).

The direct-to-LDS loads are inline assembly that set m0 themselves ("s_mov_b32 m0, sN; s_nop 0;
global_load_lds_*"); hipcc warns that it ignores m0 in their clobber lists. That is sound only while
no instruction the compiler emits reads or writes m0 (a compiler-set m0 could be overwritten by
these blocks, or one of them could leave m0 changed under a compiler use). This test compiles the
source exactly as the library is built and proves, instruction by instruction, that every m0 write
is one of those blocks and that nothing else touches m0.
"""
import os
import re
import subprocess

import pytest

from speculative_decoding_mla_split_amd import build as hip_build

SRC = os.path.join(hip_build.PKG, "csrc", "mla_verify.hip")

# instructions that read m0 implicitly (besides the direct-to-LDS loads of the asm blocks)
IMPLICIT_M0 = re.compile(r"^(s_sendmsg|s_sendmsghalt|s_ttracedata|s_movrel|v_movrel|ds_gws|ds_append|ds_consume|"
                         r"ds_read_addtid|ds_write_addtid|v_interp|lds_param_load|lds_direct_load|buffer_load\S*lds|"
                         r"buffer_store_lds|s_cbranch_g_fork)")


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("isa") / "mla_verify.s"
    flags = [f for f in hip_build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    res = subprocess.run([hipcc, *flags, "-I", hip_build.INCLUDE, "--cuda-device-only", "-S", SRC, "-o", str(out)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return [l.split(";")[0].strip() for l in out.read_text().splitlines()]


def _instructions(lines):
    return [l for l in lines if l and not l.startswith(".") and not l.endswith(":")]


def test_m0_only_set_by_direct_to_lds_blocks(device_asm):
    ins = _instructions(device_asm)
    assert ins, "no instructions"
    n_blocks = 0
    for k, l in enumerate(ins):
        op = l.split()[0]
        if "m0" in re.split(r"[\s,]+", l)[1:]:
            # the only form allowed: our block's write, immediately followed by s_nop 0 and the load
            assert re.fullmatch(r"s_mov_b32 m0, s\d+", l), f"compiler-emitted m0 use: {l}"
            assert ins[k + 1] == "s_nop 0", f"m0 write not followed by s_nop 0: {l} / {ins[k + 1]}"
            assert ins[k + 2].startswith("global_load_lds_"), f"m0 write not feeding a load: {ins[k + 2]}"
            n_blocks += 1
        if op.startswith("global_load_lds_"):
            assert re.fullmatch(r"s_mov_b32 m0, s\d+", ins[k - 2]) and ins[k - 1] == "s_nop 0", \
                f"direct-to-LDS load without its own m0 set-up: {ins[k - 2]} / {ins[k - 1]} / {l}"
        assert not IMPLICIT_M0.match(op), f"instruction that reads m0 implicitly: {l}"
    assert n_blocks > 0


def test_partial_kernels_do_not_use_scratch_inside_the_tile_loop(device_asm):
    """Spills inside the tile loop would put a scratch access (and its wait) on every tile."""
    text = "\n".join(device_asm)
    for m in re.finditer(r"^(_Z\S*verify_partial\S*):$", text, flags=re.M):
        body = text[m.end():text.index(".Lfunc_end", m.end())]
        mfma = [i.start() for i in re.finditer(r"v_mfma", body)]
        assert len(mfma) >= 68
        loop = body[mfma[0]:mfma[-1]]
        assert "scratch_" not in loop, f"scratch access inside the tile loop of {m.group(1)[:60]}"


def _vgprs(op):
    m = re.fullmatch(r"[va]\[(\d+):(\d+)\]", op)
    if m:
        return (op[0], set(range(int(m.group(1)), int(m.group(2)) + 1)))
    m = re.fullmatch(r"([va])(\d+)", op)
    return (m.group(1), {int(m.group(2))}) if m else None


def test_asm_products_settle_before_their_registers_are_touched(device_asm):
    """The score products are inline asm, so the compiler takes each as finished once issued and
    inserts no wait states after it; the matrix core writes the 16 result registers some 30 cycles
    later. Any other instruction that reads or writes those registers before the product chain has
    settled sees (or is overwritten by) the late result. This proves, for every product with a VGPR
    result, that the next instruction touching its registers is either the chain's next product
    (same registers as accumulator, which the matrix core forwards) or comes at least 24 issue slots
    later (3 x s_nop 7, as qk_settle gives; an s_nop N counts N + 1, any other instruction 1)."""
    ins = _instructions(device_asm)
    checked = 0
    for i, l in enumerate(ins):
        parts = re.split(r"[\s,]+", l)
        if not parts[0].startswith("v_mfma") or not parts[1].startswith("v["):
            continue
        dst = _vgprs(parts[1])
        slots = 0
        for j in range(i + 1, len(ins)):
            p = re.split(r"[\s,]+", ins[j])
            ops = [_vgprs(o) for o in p[1:]]
            if p[0].startswith("v_mfma") and ops[0] == dst and len(ops) > 3 and ops[3] == dst:
                break  # the chain's next product
            if any(o and o[0] == dst[0] and o[1] & dst[1] for o in ops):
                assert slots >= 24, f"{ins[j]} touches the result of {l} {slots} slots after it"
                break
            if slots >= 24:
                break
            m = re.fullmatch(r"s_nop (\d+)", ins[j])
            slots += int(m.group(1)) + 1 if m else 1
        checked += 1
    assert checked > 0
