#!/usr/bin/env python3
"""Generate the gfx950 assembly of the FP8 grouped GEMM's tall-tile main loop.

The loop is emitted as the text of one inline-asm statement (a C string
literal, one line per instruction) that `gemm_fp8.hip` includes.  Writing it
out instruction by instruction fixes what the compiler would otherwise decide:
which physical registers hold the accumulators and the weight ring (no copies
at the loop back edge), that the activation fragments of the next 16-row block
are read from LDS while the current block's matrix instructions run, that the
loads are spread between the matrix instructions instead of issued as one
burst, and exact vector-memory wait counts.

Unit tile: up to 192 or 256 rows x 256 columns, one 128-wide K block per
step, v_mfma_scale_f32_16x16x128_f8f6f4 with the power-of-two scales passed as
E8M0 exponents.  4 waves, each owning 64 columns (4 column blocks of 16) and
all 12 (16) row blocks (1 wave per SIMD, 512 registers).

The scales travel with the K pipeline instead of being staged per unit: each
ring slot of LDS holds the K block's activation rows and, after them, the
block's fp32 row scales (one global_load_lds_dword per wave: 64 rows each, the
4 waves cover 256 rows); each wave also loads its weight scale for the block
into a VGPR ring.  The exponent is the fp32 bit pattern shifted right by 23.

Register map (physical, listed as clobbers of the asm statement):
  a[0:16*rows/16-1] accumulators (block j, column block c at a[16j + 4c]);
  activation fragments (2 buffers of 8): a[192:207] for 192 rows, the 16
  VGPRs below the weight ring for 256 rows (the accumulators fill the AGPRs);
  v[256-32S:255] weight ring (S slots x 4 column blocks x 8);
  below it: per slot the two fragment addresses, the row-scale address and the
  weight-scale register; the two exponents in use, the output offset and 16
  epilogue temporaries.

Usage: python gen_fp8_asm.py OUT.inc
"""

from __future__ import annotations

import sys

CB = 4            # 16-column blocks per wave
SCALE_ROWS = 256      # row scales per slot (4 waves x 64 lanes; rows past the unit repeat its last row)


class Cfg:
    def __init__(self, rows: int, S: int, name: str):
        assert rows in (192, 256)
        self.rows, self.S, self.name = rows, S, name
        self.slot_a = rows * 128                 # activation bytes of one ring slot in LDS
        self.slot = self.slot_a + 4 * SCALE_ROWS  # bytes of one ring slot
        self.rbw = rows // 16                    # row blocks per wave at most
        self.apw = rows // 8 // 4                # 1-KB activation copies per wave per K block
        self.ops = 2 * CB + self.apw + 2         # vector-memory instructions per wave per K block
        self.wait = self.ops * (S - 2)           # outstanding once the block about to be used has landed
        assert self.wait <= 63, "vmcnt holds at most 63"
        self.wbase = 256 - 32 * S                # weight ring
        # activation fragments (2 buffers of 8): AGPRs above the accumulators while they fit
        self.frag_v = 16 * self.rbw + 16 > 256
        self.v_frag = self.wbase - 16
        self.v_alo = (self.v_frag if self.frag_v else self.wbase) - (4 * S + 20)  # fragment addresses (2 per slot)
        self.v_sadr = self.v_alo + 2 * S         # row-scale LDS address, per slot
        self.v_swr = self.v_sadr + S             # weight scale, per slot
        self.v_swe = self.v_swr + S              # weight-scale exponent
        self.v_sae = self.v_swe + 1              # row-scale exponents, 2 buffers
        self.v_doff = self.v_swe + 3             # running output offset
        self.v_t = self.v_swe + 4                # 16 epilogue temporaries
        assert self.v_alo >= 0

    def acc(self, j, c):
        return 16 * j + 4 * c

    def buf(self, b, lo=0, hi=7):
        base = (self.v_frag if self.frag_v else 16 * self.rbw) + 8 * b
        return f"{'v' if self.frag_v else 'a'}[{base + lo}:{base + hi}]"


def wrange(cfg, s, c, lo, hi):
    r = cfg.wbase + 32 * s + 8 * c
    return f"v[{r + lo}:{r + hi}]"


def issue_items(cfg, t, half):
    """The loads of one K block into ring slot t, as separate items, and the offset update after them
    (offsets advance unless the next block would be past the last one)."""
    items = []
    for c in range(CB):
        items.append([f"global_load_dwordx4 {wrange(cfg, t, c, 0, 3)}, %[wo{c}], %[wb]"])
        items.append([f"global_load_dwordx4 {wrange(cfg, t, c, 4, 7)}, %[wo{c}], %[wb] offset:{half}"])
    for i in range(cfg.apw):
        items.append([f"s_add_u32 m0, %[ma], {t * cfg.slot + i * 1024}", "s_nop 0",
                      f"global_load_lds_dwordx4 %[ao{i}], %[ab]"])
    items.append([f"s_add_u32 m0, %[ms], {t * cfg.slot}", "s_nop 0", "global_load_lds_dword %[so], %[sb]"])
    items.append([f"global_load_dword v{cfg.v_swr + t}, %[wso], %[swb]"])
    upd = ["s_add_u32 %[q], %[q], 1", "s_cmp_lt_u32 %[q], %[kb]", "s_cselect_b32 %[inc], 128, 0",
           "s_cselect_b32 %[t], %[wstep], 0", "s_cselect_b32 %[inc4], 4, 0"]
    upd += [f"v_add_u32_e32 %[wo{c}], %[t], %[wo{c}]" for c in range(CB)]
    upd += [f"v_add_u32_e32 %[ao{i}], %[inc], %[ao{i}]" for i in range(cfg.apw)]
    upd += ["v_add_u32_e32 %[so], %[inc4], %[so]", "v_add_u32_e32 %[wso], %[inc4], %[wso]"]
    return items, upd


def compute(cfg, s, t, half):
    """Multiply K block s of the ring (row blocks 0 .. rbe-1) and issue the loads of ring slot t on the
    way, one item after each row block (the rest after the last)."""
    items, upd = issue_items(cfg, t, half)
    lo, hi, sadr = cfg.v_alo + 2 * s, cfg.v_alo + 2 * s + 1, cfg.v_sadr + s
    out = [
        f"v_lshrrev_b32_e32 v{cfg.v_swe}, 23, v{cfg.v_swr + s}",
        f"ds_read_b128 {cfg.buf(0, 0, 3)}, v{lo}",
        f"ds_read_b128 {cfg.buf(0, 4, 7)}, v{hi}",
        f"ds_read_b32 v{cfg.v_sae}, v{sadr}",
        "s_waitcnt lgkmcnt(0)",
        f"v_lshrrev_b32_e32 v{cfg.v_sae}, 23, v{cfg.v_sae}",
    ]
    k = 0
    for j in range(cfg.rbw):
        b, bn = j % 2, 1 - j % 2
        out += [f"s_cmp_le_u32 %[rbe], {j}", "s_cbranch_scc1 5f"]  # no row block j: only its load item
        if j + 1 < cfg.rbw:
            out += [
                f"s_cmp_le_u32 %[rbe], {j + 1}",
                "s_cbranch_scc1 3f",
                f"ds_read_b128 {cfg.buf(bn, 0, 3)}, v{lo} offset:{(j + 1) * 2048}",
                f"ds_read_b128 {cfg.buf(bn, 4, 7)}, v{hi} offset:{(j + 1) * 2048}",
                f"ds_read_b32 v{cfg.v_sae + bn}, v{sadr} offset:{64 * (j + 1)}",
                "3:",
            ]
        out.append("s_nop 1")
        for c in range(CB):
            a0 = cfg.acc(j, c)
            out.append(f"v_mfma_scale_f32_16x16x128_f8f6f4 a[{a0}:{a0 + 3}], {wrange(cfg, s, c, 0, 7)}, "
                       f"{cfg.buf(b)}, a[{a0}:{a0 + 3}], v{cfg.v_swe}, v{cfg.v_sae + b} op_sel_hi:[0,0,0]")
        out += ["s_waitcnt lgkmcnt(0)", f"v_lshrrev_b32_e32 v{cfg.v_sae + bn}, 23, v{cfg.v_sae + bn}", "5:"]
        if k < len(items):
            out += items[k]
            k += 1
    for it in items[k:]:
        out += it
    out += upd
    return out


def step(cfg, s, last, half):
    out = [f"s_waitcnt vmcnt({cfg.wait})", "s_waitcnt lgkmcnt(0)", "s_barrier"]
    out += compute(cfg, s, (s + cfg.S - 1) % cfg.S, half)
    out += [
        "s_add_u32 %[ks], %[ks], 1",
        "s_cmp_lt_u32 %[ks], %[kb]",
        "s_cbranch_scc1 8b" if last else "s_cbranch_scc0 9f",
    ]
    return out


def epilogue(cfg):
    """bf16 stores of this wave's rows (rows >= mrows masked off); %[t] counts the rows left."""
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
        f"v_mov_b32_e32 v{cfg.v_doff}, %[doff]",
    ]
    T = cfg.v_t
    for j in range(cfg.rbw):
        out += [
            f"s_cmp_le_u32 %[rbe], {j}",
            "s_cbranch_scc1 7f",
            "v_cmp_gt_i32_e32 vcc, %[t], %[l16]",
            "s_and_saveexec_b64 %[sv], vcc",
        ]
        for c in range(CB):
            for r in range(4):
                out.append(f"v_accvgpr_read_b32 v{T + 4 * c + r}, a{cfg.acc(j, c) + r}")
        out.append("s_nop 1")
        for c in range(CB):
            p = cfg.v_alo + 2 * c
            out.append(f"v_cvt_pk_bf16_f32 v{p}, v{T + 4 * c}, v{T + 4 * c + 1}")
            out.append(f"v_cvt_pk_bf16_f32 v{p + 1}, v{T + 4 * c + 2}, v{T + 4 * c + 3}")
        out.append("s_nop 1")
        for c in range(CB):
            p = cfg.v_alo + 2 * c
            out.append(f"global_store_dwordx2 v{cfg.v_doff}, v[{p}:{p + 1}], %[db] offset:{32 * c}")
        out += [
            "s_mov_b64 exec, %[sv]",
            f"v_add_u32_e32 v{cfg.v_doff}, %[dstep], v{cfg.v_doff}",
            "s_sub_i32 %[t], %[t], 16",
        ]
    out.append("7:")
    return out


def program(cfg, half):
    S = cfg.S
    out = [f"v_mov_b32_e32 v{cfg.v_alo}, %[alo]", f"v_mov_b32_e32 v{cfg.v_alo + 1}, %[ahi]",
           f"v_mov_b32_e32 v{cfg.v_sadr}, %[sadr]"]
    for s in range(1, S):
        out.append(f"v_add_u32_e32 v{cfg.v_alo + 2 * s}, {s * cfg.slot}, %[alo]")
        out.append(f"v_add_u32_e32 v{cfg.v_alo + 2 * s + 1}, {s * cfg.slot}, %[ahi]")
        out.append(f"v_add_u32_e32 v{cfg.v_sadr + s}, {s * cfg.slot}, %[sadr]")
    out += [f"v_accvgpr_write_b32 a{r}, 0" for r in range(cfg.acc(cfg.rbw, 0))]
    out += ["s_mov_b32 %[q], 0"]
    for t in range(S - 1):
        items, upd = issue_items(cfg, t, half)
        out += [ins for it in items for ins in it] + upd
    out += ["s_mov_b32 %[ks], 0", "8:"]
    for s in range(S):
        out += step(cfg, s, s == S - 1, half)
    out += epilogue(cfg)
    return out


def clobbers(cfg):
    top = 16 * cfg.rbw + (0 if cfg.frag_v else 16)
    regs = [f'"v{r}"' for r in range(cfg.v_alo, 256)] + [f'"a{r}"' for r in range(0, top)]
    return ", ".join(regs)


CONFIGS = [Cfg(192, 4, "TALL192"), Cfg(256, 4, "TALL256")]


def main():
    out_path = sys.argv[1]
    with open(out_path, "w") as f:
        f.write("// Generated by gen_fp8_asm.py -- do not edit.\n")
        f.write(f"#define MOE_FP8_TALL_SCALE_ROWS {SCALE_ROWS}\n")
        for cfg in CONFIGS:
            n = cfg.name
            f.write(f"// {n}: {cfg.rows} rows, ring {cfg.S}, {cfg.rbw} row blocks per wave, {cfg.apw} activation "
                    f"copies and {cfg.ops} loads per wave per K block, wait {cfg.wait}\n")
            f.write(f"#define MOE_FP8_{n}_SLOT_A {cfg.slot_a}\n#define MOE_FP8_{n}_SLOT {cfg.slot}\n"
                    f"#define MOE_FP8_{n}_APW {cfg.apw}\n#define MOE_FP8_{n}_S {cfg.S}\n")
            f.write(f"#define MOE_FP8_{n}_AO_OUTS " + ", ".join(f'[ao{i}] "+v"(ao[{i}])' for i in range(cfg.apw))
                    + "\n")
            for suffix, half in (("", 64), ("_PACKED", 1024)):
                f.write(f"#define MOE_FP8_{n}_LOOP{suffix} \\\n")
                for ln in program(cfg, half):
                    f.write(f'  "{ln}\\n" \\\n')
                f.write("  \"\"\n")
            f.write(f"#define MOE_FP8_{n}_CLOBBERS {clobbers(cfg)}\n")


if __name__ == "__main__":
    main()
