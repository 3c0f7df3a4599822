"""Host checks of the generated tall-tile FP8 loop (gen_fp8_asm.py): the text the build compiles into the
kernel must keep the invariants the loop relies on.  No GPU needed."""

import importlib.util
import os
import re

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
GEN = os.path.join(HERE, "..", "int4_weights_amd", "csrc", "gen_fp8_asm.py")


@pytest.fixture(scope="module")
def gen():
    spec = importlib.util.spec_from_file_location("gen_fp8_asm", GEN)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _programs(gen):
    for cfg in gen.CONFIGS:
        for packed in (False, True):
            yield cfg, packed, gen.program(cfg, packed)


def test_every_local_label_reference_resolves(gen):
    for cfg, packed, prog in _programs(gen):
        for i, line in enumerate(prog):
            for m in re.finditer(r"\b(\d+)([fb])\b", line):
                n, d = m.group(1), m.group(2)
                span = prog[i + 1:] if d == "f" else prog[:i]
                assert f"{n}:" in span, (cfg.name, packed, i, line)


def test_wait_counts_fit_the_hardware_fields(gen):
    for cfg, packed, prog in _programs(gen):
        for line in prog:
            m = re.match(r"s_waitcnt vmcnt\((\d+)\)", line)
            if m:
                assert 0 <= int(m.group(1)) <= 63, line
            m = re.match(r"s_waitcnt lgkmcnt\((\d+)\)", line)
            if m:
                assert 0 <= int(m.group(1)) <= 15, line


def _walk(prog, rbe, kb):
    """Follow the generated control flow for one unit (row-tile count rbe, kb K blocks) and count what it
    executes: barriers, matrix instructions and vector-memory loads.  Scalar tests are evaluated for the three
    conditions the text branches on (the row-tile dispatch, kb <= 4, the loop back-edge)."""
    labels = {l[:-1]: i for i, l in enumerate(prog) if re.fullmatch(r"\d+:", l)}

    def target(ref, i):
        n, d = ref[:-1], ref[-1]
        if d == "f":
            return next(j for j in range(i + 1, len(prog)) if prog[j] == f"{n}:")
        return max(j for j in range(i) if prog[j] == f"{n}:")

    pc, scc, ks = 0, False, None
    counts = {"barrier": 0, "mfma": 0, "load": 0, "steps": 0}
    for _ in range(10_000_000):
        if pc >= len(prog):
            break
        line = prog[pc]
        if line == "s_barrier":
            counts["barrier"] += 1
        elif line.startswith("v_mfma"):
            counts["mfma"] += 1
        elif line.startswith("global_load"):
            counts["load"] += 1
        m = re.fullmatch(r"s_cmp_eq_u32 %\[rbe\], (\d+)", line)
        if m:
            scc = rbe == int(m.group(1))
        if line == "s_cmp_le_u32 %[kb], 4":
            scc = kb <= 4
        if line == "s_mov_b32 %[ks], 4":
            ks = 4
        if line == "s_add_u32 %[ks], %[ks], 4":
            ks += 4
        if line == "s_cmp_lt_u32 %[ks], %[kb]":
            scc = ks < kb
        if line == "s_cmp_eq_u32 %[won], 0":
            scc = False  # a wave with columns
        m = re.fullmatch(r"s_cbranch_scc([01]) (\d+[fb])", line)
        if m:
            if scc == (m.group(1) == "1"):
                pc = target(m.group(2), pc)
                continue
        m = re.fullmatch(r"s_branch (\d+[fb])", line)
        if m:
            pc = target(m.group(1), pc)
            continue
        pc += 1
    return counts


@pytest.mark.parametrize("kb", [4, 8, 12, 56])
def test_each_unit_path_runs_its_blocks_once(gen, kb):
    """For every row-tile count: 4 MFMAs per row tile and K block, one barrier per K block but the last, plus
    the prologue's and the epilogue's two (so all waves of a workgroup meet at the same barriers), and the
    loads of exactly kb blocks."""
    for cfg in gen.CONFIGS:
        prog = gen.program(cfg, True)
        for rbe in range(2, cfg.rt + 1):
            c = _walk(prog, rbe, kb)
            assert c["mfma"] == 4 * rbe * kb, (cfg.name, rbe, kb, c)
            assert c["barrier"] == 1 + (kb - 1) + 2, (cfg.name, rbe, kb, c)
            groups = kb // gen.GROUP
            assert c["load"] == kb * cfg.ops + groups, (cfg.name, rbe, kb, c)


def test_register_regions_do_not_overlap(gen):
    for cfg in gen.CONFIGS:
        ring = set(range(cfg.wbase, 256))
        region = set(range(cfg.v_alo, cfg.v_frag if cfg.frag_v else cfg.wbase))
        assert not ring & region
        if cfg.frag_v:
            frags = set(range(cfg.v_frag, cfg.v_frag + 16 * gen.NBUF))
            assert not frags & ring and not frags & region
        else:
            assert cfg.nacc + 16 * gen.NBUF <= 256  # fragments in the AGPRs above the accumulators
        assert cfg.v_doff < (cfg.v_frag if cfg.frag_v else cfg.wbase)
        # epilogue: two 16-register read-back buffers and 16 temporaries inside the (idle) weight ring
        assert cfg.wbase + 32 <= cfg.v_t and cfg.v_t + 16 <= 256
