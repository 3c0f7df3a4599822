"""Host checks of the generated tall-tile loops (gen_fp8_asm.py; FP8, bf16 and MXFP4 configurations): the text
the build compiles into the kernels must keep the invariants the loop relies on.  No GPU needed."""

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


def _orders(cfg):
    return (True,) if cfg.fp4 else (False, True)  # MXFP4 weights: packed order only


def _configs(gen):
    """The built configurations, plus the generator's other load distance (3) on each operand format."""
    return list(gen.CONFIGS) + [gen.Cfg(192, 4, "TALL192_D3", dist=3),
                                gen.Cfg(256, 4, "BF16_TALL256_D3", "bf16", dist=3),
                                gen.Cfg(256, 4, "FP4_TALL256_D3", "fp4", dist=3),
                                gen.Cfg(256, 4, "SWIGLU_TALL256_D3", swiglu=True, dist=3)]


def _programs(gen):
    for cfg in _configs(gen):
        for packed in _orders(cfg):
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


_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)\b)")


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        lo = int(m.group(2) if m.group(2) is not None else m.group(4))
        hi = int(m.group(3)) if m.group(3) is not None else lo
        out |= {(m.group(1), r) for r in range(lo, hi + 1)}
    return out


def _reads_writes(line):
    """Fixed registers an instruction reads and writes (operands the compiler assigns, %[...], are not
    fixed registers and are left out)."""
    line = re.sub(r"\s+(op_sel(_hi)?:\[[^\]]*\]|cbsz:\d+)", "", line)
    mnem, _, rest = line.partition(" ")
    ops = [o.strip().split()[0] for o in rest.split(",")] if rest else []
    if mnem.startswith(("global_store", "ds_write", "global_load_lds", "s_")) or not ops:
        return set().union(*map(_regs, ops)) if ops else set(), set()
    return set().union(set(), *map(_regs, ops[1:])), _regs(ops[0])


def _walk(prog, rbe, kb, pfd=False, hasnext=True, inflight=()):
    """Follow the generated control flow for one unit (row-tile count rbe, kb K blocks) and count what it
    executes: barriers, matrix instructions, vector-memory loads and stores.  Scalar tests are evaluated for
    the conditions the text branches on (the row-tile dispatch, kb <= 4, the loop back-edge; with the cross-unit
    prefetch, whether this unit's first copies were issued by the previous unit and whether a next unit follows).

    Along the way it models this wave's own counters with nothing completing before it is waited for: an
    instruction that reads or overwrites a register still targeted by a pending LDS read or vector-memory load
    fails, as does a 16th LDS operation in flight; reading an accumulator needs 18 wait states (instructions,
    s_nop N counting N + 1) after the matrix instruction that wrote it, and a matrix instruction reading a VGPR
    written by a vector ALU instruction needs 2."""
    labels = {l[:-1]: i for i, l in enumerate(prog) if re.fullmatch(r"\d+:", l)}

    def target(ref, i):
        n, d = ref[:-1], ref[-1]
        if d == "f":
            return next(j for j in range(i + 1, len(prog)) if prog[j] == f"{n}:")
        return max(j for j in range(i) if prog[j] == f"{n}:")

    pc, scc, ks = 0, False, None
    counts = {"barrier": 0, "mfma": 0, "load": 0, "store": 0, "lds_max": 0}
    lgkm, vm = [], []   # pending LDS / vector-memory operations: the registers each will write
    vm += [set(r) for r in inflight]  # loads the previous unit left in flight (pfd)
    ws = 0              # wait states so far
    mfma_w, valu_w = {}, {}
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
        elif line.startswith("global_store"):
            counts["store"] += 1
        m = re.fullmatch(r"s_waitcnt lgkmcnt\((\d+)\)", line)
        if m:
            del lgkm[:max(0, len(lgkm) - int(m.group(1)))]
        m = re.fullmatch(r"s_waitcnt vmcnt\((\d+)\)", line)
        if m:
            del vm[:max(0, len(vm) - int(m.group(1)))]
        if not re.fullmatch(r"\d+:", line):
            rd, wr = _reads_writes(line)
            pending = set().union(set(), *lgkm, *vm)
            assert not (rd | wr) & pending, (rbe, kb, pc, line, sorted((rd | wr) & pending))
            if line.startswith("v_accvgpr_read"):
                for r in rd:
                    assert ws - mfma_w.get(r, -99) >= 18, (rbe, kb, pc, line)
            if line.startswith("v_mfma"):
                for r in rd:
                    assert ws - valu_w.get(r, -99) >= 2, (rbe, kb, pc, line)
                for r in wr:
                    mfma_w[r] = ws
            elif line.startswith("v_"):
                for r in wr:
                    valu_w[r] = ws
            if line.startswith("ds_"):
                lgkm.append(wr)
                counts["lds_max"] = max(counts["lds_max"], len(lgkm))
            elif line.startswith("global_"):
                vm.append(wr)
            m = re.fullmatch(r"s_nop (\d+)", line)
            ws += int(m.group(1)) + 1 if m else 1
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
        if line == "s_bitcmp1_b32 %[fl], 0":
            scc = pfd
        if line == "s_bitcmp1_b32 %[fl], 1":
            scc = hasnext
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
    """For every row-tile count: 4 MFMAs (FP8, MXFP4; 8 bf16 ones) per row tile and K block, one barrier per K block
    but the last, plus the prologue's and the one that ends the unit (so all waves of a workgroup meet at the
    same barriers; SwiGLU: one more before its LDS writes), the loads of exactly kb blocks (rbe activation
    copies per wave and block; FP8: with one row-scale copy per 4 blocks), 4 stores (of 8 rows each) per row
    tile (SwiGLU: none, the C++ code stores), at most 15 LDS operations in flight, and no register used before
    the load or LDS read that fills it has been waited for."""
    for cfg in _configs(gen):
        for packed in _orders(cfg):
            prog = gen.program(cfg, packed)
            for rbe in range(2, cfg.rt + 1):
                for pfd, hasnext in ((False, True), (True, True), (True, False), (False, False)):
                    if not cfg.xpf and (pfd or not hasnext):
                        continue
                    inflight = []
                    if pfd:  # the previous unit's end: this unit's first weights and weight scales, in order
                        for ln in gen.next_unit_weights(cfg, packed):
                            if ln.startswith("global_load"):
                                inflight.append(_reads_writes(ln)[1])
                    c = _walk(prog, rbe, kb, pfd, hasnext, inflight)
                    assert c["mfma"] == (8 if cfg.bf16 else 4) * rbe * kb, (cfg.name, rbe, kb, c)
                    assert c["barrier"] == 1 + (kb - 1) + 1 + cfg.swiglu, (cfg.name, rbe, kb, c)
                    groups = 0 if cfg.bf16 else kb // gen.GROUP
                    loads = kb * cfg.ops_for(rbe) + groups
                    if cfg.xpf:  # the next unit's copies of its blocks 0 and 1 and its first row-scale group, and
                        # (hasnext) its weights and weight scales of those blocks; none of this unit's own loads of
                        # blocks 0 and 1 when the previous unit issued them (pfd)
                        loads += 2 * cfg.apw + 1 + (18 if hasnext else 0) - (2 * cfg.ops_for(rbe) + 1 if pfd else 0)
                    assert c["load"] == loads, (cfg.name, rbe, kb, pfd, c)
                    assert c["store"] == (0 if cfg.swiglu else 4 * rbe), (cfg.name, rbe, kb, c)
                    assert c["lds_max"] <= 15, (cfg.name, rbe, kb, c)


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
        # epilogue registers: inside weight-ring slots 0 .. 2, which the last K block does not use
        ep = [(cfg.v_rbk, 32), (cfg.v_t, 32), (cfg.v_pk, 16), (cfg.v_ep, 8)]
        used = [r for base, n in ep for r in range(base, base + n)]
        assert len(set(used)) == len(used)
        assert min(used) >= cfg.wbase and max(used) < cfg.wbase + 32 * (cfg.S - 1)


def _swiglu_epilogue_lines(prog, rbe):
    i = prog.index(f"{700 + rbe}:")
    j = prog.index("s_branch 7f", i)
    return prog[i + 1:j]


@pytest.mark.parametrize("rows", [192, 256])
def test_swiglu_staging_puts_each_value_where_the_rows_are_read(gen, rows):
    """Follow the SwiGLU epilogue's address and data registers per lane (symbolically: which accumulator each
    bf16 written to LDS came from) and check the bytes against the layout the unit's C++ code reads: row m at
    512 m, chunk c (gate values 8 c .. 8 c + 7 for c < 16, up values 8 (c - 16) .. for c >= 16) at position
    c ^ (m & 31).  Waves 0, 1 hold gate columns 64 w .. + 63 of the unit's 128 outputs, waves 2, 3 the up
    columns 64 (w - 2) ..; accumulator register r of lane L holds row L % 32 and column 8 (r / 4) +
    4 (L / 32) + r % 4 of its 32-column tile.  Every (row, gate/up, output) of the computed row tiles is
    written exactly once, inside the staging area, and nothing else is."""
    cfg = next(c for c in gen.CONFIGS if c.swiglu and c.rows == rows)
    for packed in (False, True):
        prog = gen.program(cfg, packed)
        for rbe in range(2, cfg.rt + 1):
            lines = _swiglu_epilogue_lines(prog, rbe)
            seen = {}
            for w in range(4):
                for lane in range(64):
                    l32, hh = lane % 32, lane // 32
                    epb = l32 * 512 + 16 * ((8 * w) ^ l32) + 8 * hh  # the lane's address, as the C++ code sets it
                    reg = {}
                    for ln in lines:
                        m = re.fullmatch(r"v_mov_b32_e32 v(\d+), %\[epb\]", ln)
                        if m:
                            reg[int(m.group(1))] = epb
                            continue
                        m = re.fullmatch(r"v_xor_b32_e32 v(\d+), (\d+), %\[epb\]", ln)
                        if m:
                            reg[int(m.group(1))] = epb ^ int(m.group(2))
                            continue
                        m = re.fullmatch(r"v_add_u32_e32 v(\d+), 0x10000, v(\d+)", ln)
                        if m:
                            reg[int(m.group(1))] = reg[int(m.group(2))] + 0x10000
                            continue
                        m = re.fullmatch(r"v_accvgpr_read_b32 v(\d+), a(\d+)", ln)
                        if m:
                            reg[int(m.group(1))] = ("acc", int(m.group(2)))
                            continue
                        m = re.fullmatch(r"v_cvt_pk_bf16_f32 v(\d+), v(\d+), v(\d+)", ln)
                        if m:
                            reg[int(m.group(1))] = (reg[int(m.group(2))], reg[int(m.group(3))])
                            continue
                        m = re.fullmatch(r"ds_write_b64 v(\d+), v\[(\d+):(\d+)\](?: offset:(\d+))?", ln)
                        if m:
                            p0, p1 = int(m.group(2)), int(m.group(3))
                            assert p1 == p0 + 1
                            addr = reg[int(m.group(1))] + int(m.group(4) or 0)
                            vals = [*reg[p0], *reg[p1]]
                            for k, v in enumerate(vals):
                                a = addr + 2 * k
                                assert 0 <= a < rows * 512 and a not in seen, (rbe, w, lane, ln)
                                seen[a] = (w, l32, hh, v)
                            continue
                        assert ln.startswith("s_"), ln  # nothing else touches registers or memory
            assert len(seen) == rbe * 32 * 512 // 2
            for a, (w, l32, hh, v) in seen.items():
                m, pos, within = a // 512, (a % 512) // 16, a % 16
                c = pos ^ (m & 31)
                kind, f = ("gate", 8 * c + within // 2) if c < 16 else ("up", 8 * (c - 16) + within // 2)
                _, accreg = v
                j, ct, r = accreg // 32, (accreg % 32) // 16, accreg % 16
                assert m == 32 * j + l32, (a, v)
                col = 32 * ct + 8 * (r // 4) + 4 * hh + r % 4
                assert (kind, f) == (("gate", 64 * w + col) if w < 2 else ("up", 64 * (w - 2) + col)), (a, v)
            # the C++ reads rows 0 .. 32 rbe - 1, all 32 chunks each
            assert {a // 512 for a in seen} == set(range(32 * rbe))


def test_code_between_two_loops_leaves_their_registers_alone(gen, tmp_path):
    """The plain tall loops end with the next unit's first weights and weight scales still in flight into the
    loop's registers (ring slots 0 and 1 and the weight-scale ring), and the next loop reads them: so the
    compiled kernel must not reference any of the loop's registers (v[v_alo] .. v255) outside its inline
    assembly.  Compiles gemm_fp8.hip for gfx950 to assembly text (no GPU needed) and scans every instruction
    of the plain tall kernels that the compiler wrote."""
    import subprocess
    import sys
    sys.path.insert(0, os.path.join(HERE, ".."))
    from int4_weights_amd import build as B
    gen.main.__globals__["sys"].argv = ["gen", os.path.join(B.CSRC, "gemm_fp8_tall_loop.inc")]
    gen.main()
    out = str(tmp_path / "gemm_fp8.s")
    r = subprocess.run([B.hipcc(), *B.flags(), "-S", "--cuda-device-only", os.path.join(B.CSRC, "gemm_fp8.hip"),
                        "-o", out], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    text = open(out).read().split("\n")
    cfgs = {int(c.rows): c for c in gen.CONFIGS if c.xpf}
    assert set(cfgs) == {192, 256}
    for rows, cfg in cfgs.items():
        name = f"_ZN3moe20gemm_fp8_tall_kernelILi{rows}EEEvNS_8GemmArgsE"
        start = next(i for i, ln in enumerate(text) if ln.startswith(name + ":"))
        end = next(i for i in range(start, len(text)) if text[i].startswith(f"\t.size\t{name},"))
        in_asm, seen = False, 0
        for ln in text[start:end + 1]:
            if ";;#ASMSTART" in ln:
                in_asm = True
                continue
            if ";;#ASMEND" in ln:
                in_asm = False
                continue
            code = ln.split(";")[0]
            if in_asm or not code.strip() or code.strip().startswith("."):
                continue
            seen += 1
            for m in re.finditer(r"\bv(\d+)\b", code):
                assert int(m.group(1)) < cfg.v_alo, (rows, ln)
            for m in re.finditer(r"\bv\[(\d+):(\d+)\]", code):
                assert int(m.group(2)) < cfg.v_alo, (rows, ln)
        assert seen > 100  # the kernel's own code was scanned
