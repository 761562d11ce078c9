"""Instruction checks on the gfx950 assembly of this library's own distance
kernels (CPU only; hipcc cross-compiles).

Bit-exact parity with the oracle needs every subtraction, square and
addition of the distance rounded on its own: no fused or packed fp32
multiply-add may appear in the count or tile-merge kernels.  The row
points must arrive through scalar loads (wave-uniform operands), which is
what keeps the inner loop at one VALU operation per arithmetic step.
"""
import re
import shutil

import pytest

from all_pairs_distance_amd import build

FORBIDDEN = re.compile(
    r"\b(v_(fma|fmac|mad|mac)_f32|v_pk_(fma|mul|add)_f32|v_fma_mix\w*|"
    r"v_mad_legacy_f32|v_fmac_legacy_f32|v_dot\w*)\b")


def kernel_bodies(asm: str, marker: str):
    out = {}
    for m in re.finditer(r"^(_Z\S*" + marker + r"\S*):", asm, flags=re.M):
        name = m.group(1)
        # the whole function: a kernel may end in several places (early
        # exits), so read to the assembler's end-of-function label
        end = asm.find(".Lfunc_end", m.end())
        out[name] = asm[m.end():end]
    return out


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if shutil.which(build.HIPCC) is None and not shutil.os.path.exists(build.HIPCC):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("asm")
    return {
        "count": open(build.device_assembly(str(d / "c.s"), "k_count.hip")).read(),
        "mfma": open(build.device_assembly(str(d / "f.s"), "k_count_mfma.hip")).read(),
        "merge": open(build.device_assembly(str(d / "m.s"), "k_merge.hip")).read(),
        "prune": open(build.device_assembly(str(d / "p.s"), "k_prune.hip")).read(),
    }


def _screened(name):
    # k_count<D, EDGES, PRUNED, SCREEN>: the last template flag
    return re.search(r"ELb[01]ELb[01]ELb1E", name) is not None


def test_count_kernels_have_no_fused_or_packed_fp32(asm):
    bodies = kernel_bodies(asm["count"], "7k_countI")
    # 12 widths x (edges or not) x (pruned or not), exact; the 7 widths
    # below 16 also screened (the wider ones screen on the matrix cores);
    # the 8 widths with several column points per lane also have the
    # small-set kernel (one point per lane, exact, unpruned, edges or not)
    assert len(bodies) == 48 + 28 + 16
    exact = {k: v for k, v in bodies.items() if not _screened(k)}
    assert len(exact) == 64
    for name, body in exact.items():
        bad = FORBIDDEN.findall(body)
        assert not bad, (name, bad[:3])
        assert "v_sub_f32" in body and "v_mul_f32" in body


SCREEN_ALLOWED = re.compile(r"\bv_(fma|fmac)_f32\b")


def test_screened_count_kernels(asm):
    """Screened kernels use fused multiply-adds for the screen value only;
    packed fp32 never appears, and the exact distance (separate subtract,
    multiply and add) is still there for the undecided pairs."""
    bodies = {k: v for k, v in kernel_bodies(asm["count"], "7k_countI").items()
              if _screened(k)}
    assert len(bodies) == 28
    other = re.compile(r"\b(v_pk_(fma|mul|add)_f32|v_fma_mix\w*|v_(mad|mac)_f32|"
                       r"v_mad_legacy_f32|v_fmac_legacy_f32|v_dot\w*)\b")
    for name, body in bodies.items():
        assert not other.search(body), name
        assert SCREEN_ALLOWED.search(body), name
        assert "v_sub_f32" in body and "v_mul_f32" in body, name


def test_matrix_core_screen_kernels(asm):
    """The matrix-core screen forms its values with fp32 MFMA only (no
    packed or mixed-precision arithmetic), and keeps the exact distance's
    separate subtract, multiply and add for the undecided pairs."""
    bodies = kernel_bodies(asm["mfma"], "12k_count_mfmaI")
    assert len(bodies) == 20   # widths 16, 24, 32, 48, 64 x edges x pruned
    other = re.compile(r"\b(v_pk_(fma|mul|add)_f32|v_fma_mix\w*|v_(mad|mac)_f32|"
                       r"v_mad_legacy_f32|v_fmac_legacy_f32|v_dot\w*|"
                       r"v_mfma_f32_\w+_(bf16|f16|xf32|i8|fp8|bf8)\w*)\b")
    for name, body in bodies.items():
        assert "v_mfma_f32_16x16x4_f32" in body or "v_mfma_f32_16x16x4f32" in body, name
        assert not other.search(body), name
        assert "v_sub_f32" in body and "v_mul_f32" in body, name


def test_tile_merge_kernels_have_no_fused_or_packed_fp32(asm):
    bodies = kernel_bodies(asm["merge"], "k_merge_tiles")
    # 12 widths x (direct or hoisted-norm form), plus the one-column-point-
    # per-lane form of the 8 widths (d <= 16) whose usual form holds more
    assert len(bodies) == 24 + 16
    for name, body in bodies.items():
        assert not FORBIDDEN.findall(body), name


def test_rows_are_scalar_loads(asm):
    bodies = kernel_bodies(asm["count"], "k_countILi3ELb0ELb0ELb0ELi8E")
    (body,) = bodies.values()
    assert re.search(r"s_load_dword", body)
    # the distance takes its row operand straight from an SGPR
    assert re.search(r"v_sub_f32_e32 v\d+, s\d+, v\d+", body)


def test_tile_bound_has_no_fused_fp32(asm):
    """The box-gap bound must round like the distance: no FMA either."""
    bodies = kernel_bodies(asm["prune"], "k_tile_list")
    assert len(bodies) == 1
    for name, body in bodies.items():
        assert not FORBIDDEN.findall(body), name
        assert "v_mul_f32" in body and "v_add_f32" in body


def _mask_read_too_early(body: str):
    """Sites where a v_addc_co_u32 reads an SGPR pair as its carry-in less
    than two wait states after a VALU instruction wrote that pair.  The
    compiler keeps that distance for the mask reads it schedules itself
    (v_cndmask, v_addc); hand-written add-with-carry must keep it too."""
    ins = [l.strip() for l in body.split("\n")]
    ins = [l for l in ins if l and not l.startswith((";", ".")) and not l.endswith(":")]
    bad = []
    for i, line in enumerate(ins):
        m = re.match(r"v_addc_co_u32_e64 v\d+, vcc, v\d+, (?:v\d+|0), (s\[\d+:\d+\])", line)
        if not m:
            continue
        reg, waits = m.group(1), 0
        for prev in reversed(ins[max(0, i - 6):i]):
            if prev.startswith("s_nop"):
                waits += int(prev.split()[1]) + 1
                continue
            if re.match(r"\w+ " + re.escape(reg) + ",", prev):
                if prev.startswith("v_") and waits < 2:
                    bad.append((prev, line))
                break
            waits += 1
            if waits >= 2:
                break
    return bad


def test_lane_mask_reads_keep_two_wait_states(asm):
    bodies = kernel_bodies(asm["count"], "7k_countI")
    sites = 0
    for name, body in bodies.items():
        sites += body.count("v_addc_co_u32_e64")
        bad = _mask_read_too_early(body)
        assert not bad, (name, bad[:2])
    assert sites > 0
