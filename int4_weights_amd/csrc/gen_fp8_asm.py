#!/usr/bin/env python3
"""Generate the gfx950 assembly of the FP8 grouped GEMM's tall-tile main loop.

The loop is emitted as the text of one inline-asm statement (a C string
literal, one line per instruction) that `gemm_fp8.hip` includes.  Writing it
out instruction by instruction fixes what the compiler would otherwise decide
for us: which physical registers hold the accumulators and the weight ring
(no copies at the loop back edge), that the activation fragments of the next
16-row block are read from LDS while the matrix instructions of the current
block run, and exact vector-memory wait counts.

Loads are interleaved with the matrix instructions (one load after each row
block) so the single wave of each SIMD never stalls on a burst of issues.

Tile: 4 waves x 64 columns (4 column blocks of 16) x up to 192 rows (12 row
blocks of 16), one 128-wide K block per step, v_mfma_scale_f32_16x16x128_f8f6f4
with the power-of-two scales passed as E8M0 exponents.  The row scales of the
unit are staged in LDS as exponent bytes [K block][row] before the loop, so a
step reads one byte per lane and issues no per-row scale loads.

Register map (physical, listed as clobbers of the asm statement):
  a[0:191]    accumulators, block (j, c) at a[16j + 4c : 16j + 4c + 3]
  a[192:207]  activation fragments, two buffers of 8
  v[128:255]  weight ring: S = 4 slots x 4 column blocks x 8 registers
  v[96:127]   addresses of the activation fragments per slot, scale exponents,
              epilogue temporaries

Usage: python gen_fp8_asm.py OUT.inc
"""

from __future__ import annotations

import sys

S = 4            # ring depth (K blocks): S - 1 in flight while one is multiplied
CB = 4           # 16-column blocks per wave
RBMAX = 12       # 16-row blocks per unit at most
APW = 6          # 1-KB activation copies per wave per K block (192 rows x 128 B / 4 waves)
SLOT_A = RBMAX * 16 * 128   # bytes of one activation slot in LDS
SAE_ROWS = RBMAX * 16        # bytes per K block of the staged row-scale exponents
OPS = 2 * CB + APW           # vector-memory instructions per wave per K block
WAIT = OPS * (S - 2)         # outstanding after the block about to be used has landed


def acc(j, c):
    return 16 * j + 4 * c


def wreg(s, c):
    return 128 + 32 * s + 8 * c


def buf(b):
    return 192 + 8 * b


V_ALO = 96   # v96 + 2s: fragment read address (low chunks) of slot s; v97 + 2s high chunks
V_SWE = 104  # weight-scale exponent of the current K block
V_SAE = 105  # row-scale exponents, buffers 0 and 1 (v105, v106)
V_DOFF = 108  # running output offset
V_T = 110    # epilogue temporaries v110..v125


HALF = 64  # byte offset of a column's second 64-K half (64 row-major, 1024 packed); set per program


def issue_items(t):
    """The loads of one K block into ring slot t, as separate items (lists of
    instructions), and the offset update that follows them (offsets advance
    unless the next block would be past the last one)."""
    items = []
    for c in range(CB):
        w = wreg(t, c)
        items.append([f"global_load_dwordx4 v[{w}:{w + 3}], %[wo{c}], %[wb]"])
        items.append([f"global_load_dwordx4 v[{w + 4}:{w + 7}], %[wo{c}], %[wb] offset:{HALF}"])
    for i in range(APW):
        items.append([f"s_add_u32 m0, %[ma], {t * SLOT_A + i * 1024}", "s_nop 0",
                      f"global_load_lds_dwordx4 %[ao{i}], %[ab]"])
    upd = ["s_add_u32 %[q], %[q], 1", "s_cmp_lt_u32 %[q], %[kb]", "s_cselect_b32 %[inc], 128, 0",
           "s_cselect_b32 %[t], %[wstep], 0"]
    upd += [f"v_add_u32_e32 %[wo{c}], %[t], %[wo{c}]" for c in range(CB)]
    upd += [f"v_add_u32_e32 %[ao{i}], %[inc], %[ao{i}]" for i in range(APW)]
    return items, upd


def issue(t):
    items, upd = issue_items(t)
    return [ins for it in items for ins in it] + upd


def compute(s, t):
    """Multiply K block s of the ring, row blocks 0 .. rbe-1, and issue the loads of
    ring slot t on the way: one load after each row block's matrix instructions
    (the rest after the last block), so a wave never sits in a burst of load
    issues while its matrix unit idles.  The next block's activation fragments
    are read from LDS while the current block's matrix instructions run."""
    items, upd = issue_items(t)
    lo, hi = V_ALO + 2 * s, V_ALO + 2 * s + 1
    out = [
        f"ds_read_b32 v{V_SWE}, %[swp]",
        "v_add_u32_e32 %[swp], 4, %[swp]",
        f"ds_read_b128 a[{buf(0)}:{buf(0) + 3}], v{lo}",
        f"ds_read_b128 a[{buf(0) + 4}:{buf(0) + 7}], v{hi}",
        f"ds_read_u8 v{V_SAE}, %[sep]",
        "s_waitcnt lgkmcnt(0)",
        f"v_lshrrev_b32_e32 v{V_SWE}, 23, v{V_SWE}",
    ]
    k = 0
    for j in range(RBMAX):
        b, bn = j % 2, 1 - j % 2
        out += [f"s_cmp_le_u32 %[rbe], {j}", "s_cbranch_scc1 5f"]  # no row block j: only its load item
        if j + 1 < RBMAX:
            out += [
                f"s_cmp_le_u32 %[rbe], {j + 1}",
                "s_cbranch_scc1 3f",
                f"ds_read_b128 a[{buf(bn)}:{buf(bn) + 3}], v{lo} offset:{(j + 1) * 2048}",
                f"ds_read_b128 a[{buf(bn) + 4}:{buf(bn) + 7}], v{hi} offset:{(j + 1) * 2048}",
                f"ds_read_u8 v{V_SAE + bn}, %[sep] offset:{16 * (j + 1)}",
                "3:",
            ]
        out.append("s_nop 1")
        for c in range(CB):
            a0 = acc(j, c)
            w = wreg(s, c)
            out.append(f"v_mfma_scale_f32_16x16x128_f8f6f4 a[{a0}:{a0 + 3}], v[{w}:{w + 7}], "
                       f"a[{buf(b)}:{buf(b) + 7}], a[{a0}:{a0 + 3}], v{V_SWE}, v{V_SAE + b} op_sel_hi:[0,0,0]")
        out += ["s_waitcnt lgkmcnt(0)", "5:"]
        if k < len(items):
            out += items[k]
            k += 1
    for it in items[k:]:
        out += it
    out += upd
    out.append(f"v_add_u32_e32 %[sep], {SAE_ROWS}, %[sep]")
    return out


def step(s, last):
    out = [
        f"s_waitcnt vmcnt({WAIT})",
        "s_waitcnt lgkmcnt(0)",
        "s_barrier",
    ]
    out += compute(s, (s + S - 1) % S)
    out += [
        "s_add_u32 %[ks], %[ks], 1",
        "s_cmp_lt_u32 %[ks], %[kb]",
        "s_cbranch_scc1 8b" if last else "s_cbranch_scc0 9f",
    ]
    return out


def epilogue():
    out = [
        "9:",
        "s_waitcnt vmcnt(0)",
        "s_waitcnt lgkmcnt(0)",
        "s_barrier",
        "s_nop 15",
        "s_nop 15",
        "s_cmp_eq_u32 %[won], 0",
        "s_cbranch_scc1 7f",
        "s_mov_b32 %[t], %[mrows]",
        f"v_mov_b32_e32 v{V_DOFF}, %[doff]",
    ]
    for j in range(RBMAX):
        out += [
            f"s_cmp_le_u32 %[rbe], {j}",
            "s_cbranch_scc1 7f",
            "v_cmp_gt_i32_e32 vcc, %[t], %[l16]",
            "s_and_saveexec_b64 %[sv], vcc",
        ]
        for c in range(CB):
            for r in range(4):
                out.append(f"v_accvgpr_read_b32 v{V_T + 4 * c + r}, a{acc(j, c) + r}")
        out.append("s_nop 1")
        for c in range(CB):
            out.append(f"v_cvt_pk_bf16_f32 v{V_ALO + 2 * c}, v{V_T + 4 * c}, v{V_T + 4 * c + 1}")
            out.append(f"v_cvt_pk_bf16_f32 v{V_ALO + 2 * c + 1}, v{V_T + 4 * c + 2}, v{V_T + 4 * c + 3}")
        out.append("s_nop 1")
        for c in range(CB):
            out.append(f"global_store_dwordx2 v{V_DOFF}, v[{V_ALO + 2 * c}:{V_ALO + 2 * c + 1}], %[db] offset:{32 * c}")
        out += [
            "s_mov_b64 exec, %[sv]",
            f"v_add_u32_e32 v{V_DOFF}, %[dstep], v{V_DOFF}",
            "s_sub_i32 %[t], %[t], 16",
        ]
    out.append("7:")
    return out


def program():
    out = [f"v_mov_b32_e32 v{V_ALO}, %[alo]", f"v_mov_b32_e32 v{V_ALO + 1}, %[ahi]"]
    for s in range(1, S):
        out.append(f"v_add_u32_e32 v{V_ALO + 2 * s}, {s * SLOT_A}, %[alo]")
        out.append(f"v_add_u32_e32 v{V_ALO + 2 * s + 1}, {s * SLOT_A}, %[ahi]")
    out += [f"v_accvgpr_write_b32 a{r}, 0" for r in range(acc(RBMAX, 0))]
    out += ["s_mov_b32 %[q], 0"]
    for t in range(S - 1):
        out += issue(t)
    out += ["s_mov_b32 %[ks], 0", "8:"]
    for s in range(S):
        out += step(s, s == S - 1)
    out += epilogue()
    return out


def clobbers():
    regs = [f'"v{r}"' for r in range(96, 256)] + [f'"a{r}"' for r in range(0, 208)]
    return ", ".join(regs)


def main():
    out_path = sys.argv[1]
    global HALF
    with open(out_path, "w") as f:
        f.write("// Generated by gen_fp8_asm.py -- do not edit.\n")
        f.write(f"// tall FP8 tile: S={S} CB={CB} RBMAX={RBMAX} APW={APW} OPS={OPS} WAIT={WAIT}\n")
        for name, half in (("MOE_FP8_TALL_LOOP", 64), ("MOE_FP8_TALL_LOOP_PACKED", 1024)):
            HALF = half
            f.write(f"#define {name} \\\n")
            for ln in program():
                f.write(f'  "{ln}\\n" \\\n')
            f.write("  \"\"\n")
        f.write(f"#define MOE_FP8_TALL_CLOBBERS {clobbers()}\n")
        f.write(f"#define MOE_FP8_TALL_S {S}\n#define MOE_FP8_TALL_RB {RBMAX}\n#define MOE_FP8_TALL_APW {APW}\n")
        f.write(f"#define MOE_FP8_TALL_SLOT_A {SLOT_A}\n#define MOE_FP8_TALL_SAE_ROWS {SAE_ROWS}\n")


if __name__ == "__main__":
    main()
