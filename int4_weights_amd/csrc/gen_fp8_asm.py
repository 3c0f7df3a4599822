#!/usr/bin/env python3
"""Generate the gfx950 assembly of the FP8 grouped GEMM's tall-tile main loop.

The loop is emitted as the text of one inline-asm statement (a C string
literal, one line per instruction) that `gemm_fp8.hip` includes.  Writing it
out instruction by instruction fixes what the compiler would otherwise decide:
which physical registers hold the accumulators and the weight ring (no copies
at the loop back edge), that the activation fragments of the next 32-row tile
are read from LDS while the current tile's matrix instructions run, that the
loads are spread between the matrix instructions instead of issued as one
burst, and exact vector-memory wait counts.

Unit tile: up to 192 or 256 rows x 256 columns, one 128-wide K block per
step, v_mfma_scale_f32_32x32x64_f8f6f4 (two per K block and 32 x 32 output
tile) with the power-of-two scales passed as E8M0 exponents; it issues at full
rate from one wave per SIMD.  4 waves, each owning 64 columns (2 column tiles
of 32) and all 6 (8) row tiles of 32 (1 wave per SIMD, 512 registers).

Operands.  The weights are the instruction's A operand, the activations its B
operand.  Both use the same assignment of K to lanes and bytes: lane L
(row L % 32, half h = L / 32) of instruction kk supplies the 32 values
k = 64 kk + 32 h .. +31 of its row, as two 16-byte pieces p (k + 16 p).  In
the packed weight order a piece is the 16-byte chunk of lane
(L % 16) + 16 (2h + p) of the row's 16-column block, half kk; activations are
read from LDS as chunks 4 kk + 2 h + p of the row.  The accumulator of lane L,
register r, holds output row L % 32 and weight column
8 (r / 4) + 4 h + r % 4 of the tile, so each lane stores 4 consecutive columns
(8 bytes) per register group.

The scales travel with the K pipeline instead of being staged per unit: each
ring slot of LDS holds the K block's activation rows and, after them, the
block's fp32 row scales (one global_load_lds_dword per wave: 64 rows each, the
4 waves cover 256 rows); each wave also loads its weight scale for the block
into a VGPR ring.  The exponent is the fp32 bit pattern shifted right by 23.

Activation copies.  A unit of rbe row tiles copies only the 32 rbe rows it computes: copy i of wave w moves
rows 8 (4 i + w) .. +7 of the K block (1 KB) into the ring slot, so each loop body issues rbe copies per wave
and K block, with its own wait counts and its own prologue.

Pipeline.  Step ks multiplies K block ks and issues the loads of block ks + dist
(dist = 2: one block in flight beyond the next, about 64 KB per CU; 3 was no
faster on HBM-bound shapes and 1-2% slower on the Qwen3-shaped ones, as a plain
streaming read also slows down with more bytes in flight).  The barrier that publishes block ks + 1 sits
inside step ks, after the fragments of the step's last row tile have been read
into registers: from then on no wave reads slot ks, so row tile 0 of block
ks + 1 (and its row scale) is read into a third fragment buffer while the last
row tile's matrix instructions run, and the next step starts without an LDS
round trip.  A unit always computes at least two row tiles (the surplus rows
repeat the last valid row and are never stored), so that barrier always has a
row tile after it.  The loop is emitted once per row-tile count (2 .. 6 or 8):
a unit jumps to its body once, and no branch sits between the matrix
instructions of a step (with one wave per SIMD a taken branch at every row
tile left the matrix pipe idle; the branch-free bodies are 4-9% faster).  The
loop's last iteration is emitted apart (it issues only block kb - 1 and waits
for fewer loads), so the main loop's only branch is its back-edge, and a
unit's first step is emitted apart too: its matrix instructions add to 0, so
the accumulators are never zeroed.  The unit's last K block issues none of the
unit's own loads and leaves ring slots 0 .. 2 idle, so the epilogue runs inside
it: while row tile j is multiplied, row tile j - 1 is converted to bf16 and
staged through the wave's 4 KB of LDS slot 0 (slot 2 with the cross-unit
pipeline, xpf, whose last two steps issue the next unit's copies of its blocks
0 and 1 into slots 0 and 1, and whose loop ends by issuing that unit's weights
of those blocks), and row tile j - 2 is stored as whole 128-byte rows; after the
loop only the last row tile remains.

Register map (physical, listed as clobbers of the asm statement):
  a[0:rows-1] accumulators (row tile j, column tile ct at a[32j + 16ct]);
  activation fragments (3 buffers of 16; row tile 0 in buffer 2, tile j >= 1 in
  buffer j % 2): a[192:239] for 192 rows, the 48 VGPRs below the weight ring
  for 256 rows (the accumulators fill the AGPRs);
  v[256-32S:255] weight ring (S slots x 2 column tiles x 2 halves x 8);
  below it: per slot the four fragment addresses, the row-scale address and
  the weight-scale register; the weight exponent, one row-scale exponent per
  fragment buffer and the output offset.  The epilogue uses weight-ring slots
  0 .. 2, idle in the last K block: two 16-register buffers for the rows read
  back from LDS, 32 temporaries, 16 packed bf16 pairs and 8 LDS addresses.

SwiGLU variant (up-projection with the activation fused): the unit's waves 0, 1 take 128 gate columns and
waves 2, 3 the 128 up columns of the same outputs; after the loop the bf16-rounded accumulators of every row
tile go to LDS, and the unit's C++ code computes silu(gate) * up and its 1x128 quantisation from there.

Usage: python gen_fp8_asm.py OUT.inc
"""

from __future__ import annotations

import sys

NBUF = 3          # activation fragment buffers (row tile 0 of the next block is read into its own)
SCALE_ROWS = 256  # rows of a scale group (4 waves x 64 lanes; rows past the unit repeat its last row)
GROUP = 4         # K blocks per row-scale copy (one 16-byte copy per row)


class Cfg:
    def __init__(self, rows: int, S: int, name: str, dtype: str = "fp8", wnt: bool = False, dist: int = 2,
                 swiglu: bool = False, xpf: bool = False):
        assert rows in (192, 256) and dtype in ("fp8", "bf16", "fp4") and not (swiglu and dtype != "fp8")
        self.swiglu = swiglu                      # epilogue: gate and up columns to LDS for SwiGLU (no stores)
        # the last K block issues the next unit's activation and row-scale copies of its blocks 0 and 1 (ring slots
        # 0 and 1, idle by then); the epilogue stages through slot 2 instead of slot 0
        self.xpf = xpf
        assert not xpf or (dtype == "fp8" and not swiglu and dist == 2)
        self.rows, self.S, self.name = rows, S, name
        self.wnt = wnt                            # weight loads nontemporal (each weight byte read by one unit)
        assert dist in (2, 3)
        self.dist = dist                          # step ks issues the loads of block ks + dist
        self.bf16 = dtype == "bf16"               # bf16 operands: four 32x32x16 instructions per 128-byte step,
        # no scales
        self.fp4 = dtype == "fp4"                 # MXFP4 weights (packed order only): 16 bytes per lane and K half,
        # one E8M0 scale per 32 K values and lane (two scale dwords per K block, shifted per lane)
        assert S == GROUP, "the unrolled loop body is one scale group"
        self.slot_a = rows * 128                 # activation bytes of one ring slot in LDS
        self.slot = self.slot_a                   # bytes of one ring slot
        self.sc_off = S * self.slot               # (fp8) two scale-group buffers of SCALE_ROWS x 16 bytes follow
        self.lds = self.sc_off + (0 if self.bf16 else 2 * SCALE_ROWS * 16)
        self.rt = rows // 32                      # 32-row tiles per unit at most
        self.apw = rows // 32                     # 1-KB activation copies per wave per K block at most (a unit of
        # rbe row tiles issues rbe: copy i of wave w is rows 8 (4 i + w) .. +7)
        self.nsw = 0 if self.bf16 else (2 if self.fp4 else 1)  # weight-scale loads per K block
        self.ops = self.ops_for(self.apw)          # vector-memory instructions per wave per K block, at most
        # (+1 more for the blocks that start a row-scale group)
        assert 2 * self.ops + 2 <= 63, "vmcnt holds at most 63"
        self.wbase = 256 - 32 * S
        self.nacc = 32 * self.rt
        self.frag_v = self.nacc + 16 * NBUF > 256
        self.v_frag = self.wbase - 16 * NBUF
        nsw = max(1, self.nsw)
        nlo = 4 * S + S + nsw * S + nsw + NBUF + 1
        self.v_alo = (self.v_frag if self.frag_v else self.wbase) - (nlo + nlo % 2)  # even: 64-bit pairs
        self.v_aadr = self.v_alo                  # slot s, (kk, p): v_aadr + 4s + 2kk + p
        self.v_sadr = self.v_alo + 4 * S
        self.v_swr = self.v_sadr + S              # weight-scale ring: slot s (and fp4 K half kk) at v_swr + nsw s + kk
        self.v_swe = self.v_swr + nsw * S         # the block's weight exponent(s): fp4 K half kk at v_swe + kk
        self.v_sae = self.v_swe + nsw             # one per fragment buffer
        self.v_doff = self.v_sae + NBUF
        assert self.v_alo >= 0
        # epilogue registers, in weight-ring slots 0 .. 2 (idle during the last K block, which uses slot 3):
        # two 16-register read-back buffers, 32 temporaries, 16 packed bf16 pairs, 8 LDS chunk addresses
        self.v_rbk = self.wbase
        self.v_t = self.wbase + 32
        self.v_pk = self.wbase + 64
        self.v_ep = self.wbase + 80
        assert self.v_ep + 8 <= self.wbase + 32 * (S - 1)
        # each wave stages one 32-row tile of bf16 (32 x 128 bytes) in its 4 KB of ring slot 0 (xpf: slot 2)
        assert 4 * 4096 <= self.slot

    def acc(self, j, ct):
        return 32 * j + 16 * ct

    def ops_for(self, rbe):
        """Vector-memory instructions per wave per K block for units of rbe row tiles (rbe activation copies)."""
        return (4 if self.fp4 else 8) + rbe + self.nsw

    def wait_at(self, s, issued, ops):
        """Loads allowed outstanding at the barrier of step s (K block ks = s mod S) that publishes block
        ks + 1: those of the blocks issued after it in earlier steps (ks + 2 when dist = 3, plus one if it
        starts a scale group; none when dist = 2) and the `issued` loads of block ks + dist this step has
        issued so far."""
        if self.dist == 2:
            return issued
        return ops + (1 if (s + 2) % GROUP == 0 and not self.bf16 else 0) + issued

    @staticmethod
    def bufid(j):
        """Fragment buffer of row tile j: buffer 2 for tile 0 (filled before the step starts), then 1, 0, ..."""
        return 2 if j == 0 else j % 2

    def buf(self, b, kk, lo=0, hi=7):
        base = (self.v_frag if self.frag_v else self.nacc) + 16 * b + 8 * kk
        return f"{'v' if self.frag_v else 'a'}[{base + lo}:{base + hi}]"


def wreg(cfg, s, ct, kk, lo, hi):
    r = cfg.wbase + 32 * s + 16 * ct + 8 * kk
    return f"v[{r + lo}:{r + hi}]"


def issue_items(cfg, t, packed, rbe):
    """The loads of one K block into ring slot t, as separate items, and the offset update after them
    (offsets advance unless the next block would be past the last one).  Block t mod S == 0 starts a scale
    group: one 16-byte copy per row of the group's 4 row scales into the group buffer %[msg] points at
    (the buffers alternate), its offset advancing unless the next group would be past the last block."""
    items = []
    for ct in range(2):
        for kk in range(2):
            if cfg.fp4:  # E2M1: 16 bytes per lane and K half (packed: chunk 2 kk + h of the column's 1 KB fragment)
                assert packed
                items.append([f"global_load_dwordx4 {wreg(cfg, t, ct, kk, 0, 3)}, %[wo{ct}], %[wb] offset:{512 * kk}"
                              + (" nt" if cfg.wnt else "")])
                continue
            for p in range(2):
                off = kk * 1024 + p * 256 if packed else kk * 64 + p * 16
                items.append([f"global_load_dwordx4 {wreg(cfg, t, ct, kk, 4 * p, 4 * p + 3)}, %[wo{ct}], %[wb] "
                              f"offset:{off}" + (" nt" if cfg.wnt else "")])
    for i in range(rbe):  # rows 8 (4 i + w) .. +7 of the slot for wave w: the unit's rbe row tiles, no more
        items.append([f"s_add_u32 m0, %[ma], {t * cfg.slot + i * 4096}", "s_nop 0",
                      f"global_load_lds_dwordx4 %[ao{i}], %[ab]"])
    upd = []
    if cfg.bf16:  # no scales: only the weight and activation offsets advance
        upd += ["s_add_u32 %[q], %[q], 1", "s_cmp_lt_u32 %[q], %[kb]", "s_cselect_b32 %[inc], 128, 0",
                "s_cselect_b32 %[t], %[wstep], 0"]
        upd += [f"v_add_u32_e32 %[wo{ct}], %[t], %[wo{ct}]" for ct in range(2)]
        upd += [f"v_add_u32_e32 %[ao{i}], %[inc], %[ao{i}]" for i in range(rbe)]
        return items, upd
    if cfg.fp4:  # the scale dwords of K halves 0 and 1 (block 2 kk + h of the lane's 16-column group)
        items += [[f"global_load_dword v{cfg.v_swr + 2 * t + kk}, %[wso], %[swb]" + (" offset:128" if kk else "")]
                  for kk in range(2)]
    else:
        items.append([f"global_load_dword v{cfg.v_swr + t}, %[wso], %[swb]"])
    if t % GROUP == 0:
        items.append(["s_mov_b32 m0, %[msg]", "s_nop 0", "global_load_lds_dwordx4 %[so], %[sb]"])
        upd += ["s_xor_b32 %[msg], %[msg], " + str(SCALE_ROWS * 16), f"s_add_u32 %[t], %[q], {GROUP}",
                "s_cmp_lt_u32 %[t], %[kb]", "s_cselect_b32 %[inc4], 16, 0", "v_add_u32_e32 %[so], %[inc4], %[so]"]
    upd += ["s_add_u32 %[q], %[q], 1", "s_cmp_lt_u32 %[q], %[kb]", "s_cselect_b32 %[inc], 128, 0",
           "s_cselect_b32 %[t], %[wstep], 0", "s_cselect_b32 %[inc4], " + ("%[sstep]" if cfg.fp4 else "4") + ", 0"]
    upd += [f"v_add_u32_e32 %[wo{ct}], %[t], %[wo{ct}]" for ct in range(2)]
    upd += [f"v_add_u32_e32 %[ao{i}], %[inc], %[ao{i}]" for i in range(rbe)]
    upd += ["v_add_u32_e32 %[wso], %[inc4], %[wso]"]
    return items, upd


def prefetch_items(cfg, nb):
    """The next unit's activation copies of its K block nb (0 or 1) into ring slot nb: all apw copies per wave
    (rows past that unit's end repeat its last row); with block 0 also its first row-scale group into the group
    buffer %[msg] points at, which then alternates as for the unit's own groups.

    The copy offsets reuse %[ao*], idle once the unit's last block is issued: copy i of the next unit reads
    row min(r_i, m - 1) (m its rows), chunk c, i.e. min(%[uo0] + 32 i K, (m - 1) K + c) with %[uo0] the
    unclamped offset r_0 K + c (c, the lane's chunk, is the same for every copy), computed with two registers of
    ring slot 0 (idle in the last K block until its epilogue uses it) before the first copy.  For block 1 each
    offset first advances by 128 bytes: an instruction offset would move the copy's LDS destination as well."""
    T, U = cfg.wbase, cfg.wbase + 1
    items = [([f"v_add_u32_e32 %[ao{i}], 128, %[ao{i}]"] if nb else [])
             + [f"s_add_u32 m0, %[ma], {nb * cfg.slot + i * 4096}", "s_nop 0",
                f"global_load_lds_dwordx4 %[ao{i}], %[nab]"] for i in range(cfg.apw)]
    if nb == 0:
        # (%[t] = 32 K, free in the last K block)
        setup = ["s_lshl_b32 %[t], %[kb], 12", f"v_add_u32_e32 v{T}, %[nlim], %[cc]", f"v_mov_b32_e32 v{U}, %[uo0]"]
        for i in range(cfg.apw):
            setup += [f"v_min_u32_e32 %[ao{i}], v{U}, v{T}"] + ([f"v_add_u32_e32 v{U}, %[t], v{U}"]
                                                               if i + 1 < cfg.apw else [])
        items[0] = setup + items[0]
        items.append(["s_mov_b32 m0, %[msg]", "s_nop 0", "global_load_lds_dwordx4 %[nso], %[nsb]",
                      f"s_xor_b32 %[msg], %[msg], {SCALE_ROWS * 16}"])
    return items


def weight_exponents(cfg, s):
    """The weight scale exponents of ring slot s: the fp32 scale's bit pattern shifted right by 23 (FP8), or
    (fp4) each K half's scale dword shifted right by 8 (l32 / 16) bytes, so that byte 2 ct is the scale of the
    lane's column in column tile ct."""
    if cfg.fp4:
        return [f"v_lshrrev_b32_e32 v{cfg.v_swe + kk}, %[fsh], v{cfg.v_swr + 2 * s + kk}" for kk in range(2)]
    return [f"v_lshrrev_b32_e32 v{cfg.v_swe}, 23, v{cfg.v_swr + s}"]


def frag_reads(cfg, s, b, j):
    """LDS reads of row tile j's activation fragments (both halves kk, both pieces p) into buffer b."""
    out = []
    for kk in range(2):
        for p in range(2):
            off = f" offset:{j * 4096}" if j else ""
            out.append(f"ds_read_b128 {cfg.buf(b, kk, 4 * p, 4 * p + 3)}, v{cfg.v_aadr + 4 * s + 2 * kk + p}{off}")
    return out


def publish(cfg, s, wait):
    """The barrier of step s that publishes K block ks + 1, placed after the fragments of the step's last
    row tile are in registers: wait until at most `wait` loads are outstanding (this wave's loads of block
    ks + 1 have landed), barrier (every wave's copies of the block have landed and every wave has read all of
    slot s), then read row tile 0 of block ks + 1 and its row scale into buffer 2 while the last row tile's
    matrix instructions run."""
    sn = (s + 1) % cfg.S
    out = [f"s_waitcnt vmcnt({wait})", "s_barrier"]
    if s == cfg.S - 1 and not cfg.bf16:  # block ks + 1 opens the next scale group, in the other group buffer
        out.append(f"v_xor_b32_e32 v{cfg.v_sadr}, {SCALE_ROWS * 16}, v{cfg.v_sadr}")
    out += frag_reads(cfg, sn, 2, 0)
    if not cfg.bf16:
        out.append(f"ds_read_b32 v{cfg.v_sae + 2}, v{cfg.v_sadr}" + (f" offset:{4 * sn}" if sn else ""))
    return out


def mfma(cfg, s, b, j, ct, kk, src_zero):
    """The matrix instructions of K half kk for row tile j (fragment buffer b) and column tile ct: one scaled
    32x32x64 FP8 instruction, or two 32x32x16 bf16 ones on the two 16-byte pieces of each operand (the same K
    values in both operands, so the products match), the second accumulating onto the first."""
    a0 = cfg.acc(j, ct)
    acc = f"a[{a0}:{a0 + 15}]"
    if cfg.fp4:  # E2M1 A operand (cbsz 4), 4 registers; scale byte 2 ct of the lane's shifted scale dword
        return [f"v_mfma_scale_f32_32x32x64_f8f6f4 {acc}, {wreg(cfg, s, ct, kk, 0, 3)}, {cfg.buf(b, kk)}, "
                f"{'0' if src_zero else acc}, v{cfg.v_swe + kk}, v{cfg.v_sae + b} op_sel_hi:[{ct},0,0] cbsz:4"]
    if not cfg.bf16:
        return [f"v_mfma_scale_f32_32x32x64_f8f6f4 {acc}, {wreg(cfg, s, ct, kk, 0, 7)}, {cfg.buf(b, kk)}, "
                f"{'0' if src_zero else acc}, v{cfg.v_swe}, v{cfg.v_sae + b} op_sel_hi:[0,0,0]"]
    return [f"v_mfma_f32_32x32x16_bf16 {acc}, {wreg(cfg, s, ct, kk, 4 * p, 4 * p + 3)}, "
            f"{cfg.buf(b, kk, 4 * p, 4 * p + 3)}, {'0' if src_zero and p == 0 else acc}" for p in range(2)]


def compute(cfg, s, t, packed, rbe, final=False, first=False):
    """Multiply K block s of the ring (row tiles 0 .. rbe-1; rbe >= 2 is fixed for the body, so the code has no
    branch between matrix instructions) and issue the loads of ring slot t (block ks + dist) on the way, one item
    after each of the evenly spaced matrix instructions (a burst of loads stalls every wave on the shared load
    path).  Row tile 0's fragments and row scale were read into buffer 2 by the previous step; the barrier that
    publishes the next block sits after row tile rbe - 2 (publish).

    final: step s of the loop's last iteration (K blocks kb-4 .. kb-1).  Steps 0 .. 3 - dist still issue
    blocks up to kb - 1, the later ones issue nothing, so their waits are for fewer loads (step 2: none), and
    step 3 has no next block to publish (it carries the bf16 epilogue, except with SwiGLU).

    first: the unit's first K block; each accumulator's first matrix instruction adds to 0 instead of the
    accumulator, so the accumulators need no zeroing."""
    if final and s == cfg.S - 1 and not cfg.swiglu:
        return compute_last(cfg, s, rbe)
    items, upd = issue_items(cfg, t, packed, rbe)
    if final and s > cfg.S - 1 - cfg.dist:  # its block would be past the last one
        items, upd = (prefetch_items(cfg, 0) if cfg.xpf and s == cfg.S - 2 else []), []
    nslots = 4 * rbe
    place = [[] for _ in range(nslots)]  # matrix-instruction slot -> the items issued right after it
    for i, it in enumerate(items):
        place[(i * nslots) // len(items)].append(it)
    sadr = cfg.v_sadr  # row r's scale of K block s of the group at r * 16 + 4 s
    out = (["s_waitcnt lgkmcnt(0)"] if cfg.bf16 else
           weight_exponents(cfg, s) + ["s_waitcnt lgkmcnt(0)",
                                       f"v_lshrrev_b32_e32 v{cfg.v_sae + 2}, 23, v{cfg.v_sae + 2}"])
    for j in range(rbe):
        b = cfg.bufid(j)
        if j + 1 < rbe:
            bn = cfg.bufid(j + 1)
            out += frag_reads(cfg, s, bn, j + 1)
            if not cfg.bf16:
                out.append(f"ds_read_b32 v{cfg.v_sae + bn}, v{sadr} offset:{512 * (j + 1) + 4 * s}")
        out.append("s_nop 1")
        q = 0
        for kk in range(2):  # consecutive instructions write different accumulators
            for ct in range(2):
                out += mfma(cfg, s, b, j, ct, kk, first and kk == 0)
                out += [ins for it in place[4 * j + q] for ins in it]
                q += 1
        if j + 1 < rbe:
            out += ["s_waitcnt lgkmcnt(0)"] + ([] if cfg.bf16 else
                                               [f"v_lshrrev_b32_e32 v{cfg.v_sae + bn}, 23, v{cfg.v_sae + bn}"])
            if j + 2 == rbe and not (final and s == cfg.S - 1):  # row tile j + 1 is the last one
                issued = sum(len(place[i]) for i in range(4 * (j + 1)))
                wait = issued if final and s == cfg.S - 2 else cfg.wait_at(s, issued, cfg.ops_for(rbe))
                out += publish(cfg, s, wait)
    out += upd
    return out


def body(cfg, packed, rbe):
    """The K loop for units of rbe row tiles: iterations of S steps (one per ring slot, S = 4 K blocks); all
    but the last issue the loads of the block dist ahead in every step, the last one (final) is emitted apart.
    The unit's first step (accumulating onto 0) is emitted once more for either kind of iteration and then
    joins the loop at its second step."""
    head, mid, fin, fin_mid, first_fin = 200 + rbe, 300 + rbe, 400 + rbe, 500 + rbe, 600 + rbe
    t0 = cfg.dist  # ring slot of the loads issued by step 0
    out = ["s_cmp_le_u32 %[kb], 4", f"s_cbranch_scc1 {first_fin}f", "s_mov_b32 %[ks], 4"]
    out += compute(cfg, 0, t0, packed, rbe, first=True) + [f"s_branch {mid}f", f"{head}:"]
    out += compute(cfg, 0, t0, packed, rbe) + [f"{mid}:"]
    for s in range(1, cfg.S):
        out += compute(cfg, s, (s + cfg.dist) % cfg.S, packed, rbe)
    out += ["s_add_u32 %[ks], %[ks], 4", "s_cmp_lt_u32 %[ks], %[kb]", f"s_cbranch_scc1 {head}b", f"s_branch {fin}f",
            f"{first_fin}:"]
    out += compute(cfg, 0, t0, packed, rbe, final=True, first=True) + [f"s_branch {fin_mid}f", f"{fin}:"]
    out += compute(cfg, 0, t0, packed, rbe, final=True) + [f"{fin_mid}:"]
    for s in range(1, cfg.S):
        out += compute(cfg, s, (s + cfg.dist) % cfg.S, packed, rbe, final=True)
    out.append(f"s_branch {700 + rbe}f")
    return out


def ep_setup(cfg):
    """Output offset, rows left, and the LDS address of each logical 16-byte chunk c of this lane's staged row
    (row m at m*128 of the wave's 4 KB, chunk c at position c ^ (m & 7), plus the lane's 8-byte half): %[epb]
    is chunk 0's, and the XOR flips the position bits."""
    E = cfg.v_ep
    return ([f"v_mov_b32_e32 v{cfg.v_doff}, %[doff]", "s_mov_b32 %[t], %[mrows]", f"v_mov_b32_e32 v{E}, %[epb]"]
            + [f"v_xor_b32_e32 v{E + c}, {16 * c}, %[epb]" for c in range(1, 8)])


def ep_convert(cfg, j, ct):
    """Row tile j, column tile ct: accumulators to 8 packed bf16 pairs (RNE)."""
    T = cfg.v_t + 16 * ct
    out = [f"v_accvgpr_read_b32 v{T + r}, a{cfg.acc(j, ct) + r}" for r in range(16)] + ["s_nop 1"]
    for g in range(4):
        pr = cfg.v_pk + 8 * ct + 2 * g
        out += [f"v_cvt_pk_bf16_f32 v{pr}, v{T + 4 * g}, v{T + 4 * g + 1}",
                f"v_cvt_pk_bf16_f32 v{pr + 1}, v{T + 4 * g + 2}, v{T + 4 * g + 3}"]
    return out


def ep_stage(cfg, j):
    """Write row tile j's bf16 rows to the wave's staging area and read them back as 16 bytes per lane, 8 lanes
    per 128-byte row, into read-back buffer j % 2 (LDS operations of one wave complete in order)."""
    out = [f"ds_write_b64 v{cfg.v_ep + 4 * ct + g}, v[{cfg.v_pk + 8 * ct + 2 * g}:{cfg.v_pk + 8 * ct + 2 * g + 1}]"
           for ct in range(2) for g in range(4)]
    for q in range(4):
        r = cfg.v_rbk + 16 * (j % 2) + 4 * q
        out.append(f"ds_read_b128 v[{r}:{r + 3}], %[rb]" + (f" offset:{1024 * q}" if q else ""))
    return out


def ep_store_full(cfg, j):
    """Row tile j, all 32 rows valid: 8 whole 128-byte rows per store (none from a wave without columns)."""
    out = ["s_and_saveexec_b64 %[sv], %[wm]"]
    for q in range(4):
        r = cfg.v_rbk + 16 * (j % 2) + 4 * q
        out += [f"global_store_dwordx4 v{cfg.v_doff}, v[{r}:{r + 3}], %[db] nt",
                f"v_add_u32_e32 v{cfg.v_doff}, %[dstep], v{cfg.v_doff}"]
    return out + ["s_mov_b64 exec, %[sv]", "s_sub_i32 %[t], %[t], 32", "s_nop 1"]


def ep_store_masked(cfg, j):
    """Row tile j's 4 groups of 8 rows, rows at or past the unit's end masked off (%[t] counts the rows left)."""
    out = []
    for q in range(4):
        r = cfg.v_rbk + 16 * (j % 2) + 4 * q
        out += ["v_cmp_gt_i32_e32 vcc, %[t], %[l8]", "s_and_saveexec_b64 %[sv], vcc",
                f"global_store_dwordx4 v{cfg.v_doff}, v[{r}:{r + 3}], %[db] nt", "s_mov_b64 exec, %[sv]",
                f"v_add_u32_e32 v{cfg.v_doff}, %[dstep], v{cfg.v_doff}", "s_sub_i32 %[t], %[t], 8"]
    return out


def compute_last(cfg, s, rbe):
    """The unit's last K block (ring slot s = S - 1 of the final iteration), with the epilogue folded in.

    None of the unit's own loads are issued and no block is published, so ring slots 0 .. 2 are idle: while row
    tile j is multiplied, row tile j - 1 (final since the previous row tile's matrix instructions) is
    converted to bf16 and staged through the wave's 4 KB of slot 0 (xpf: slot 2, the next unit's block 1
    copies being issued meanwhile), and row tile j - 2, read back in the
    previous row tile, is stored as whole 128-byte rows.  All rows of the row tiles stored here are valid
    (only the last row tile, and row tile 0 of a two-tile unit, can be partial; both are stored by the
    epilogue after the loop).  Row tile j + 1's fragments are read after row tile j's first matrix
    instruction, and the LDS operations in flight stay within the 15 that lgkmcnt counts."""
    out = (["s_waitcnt lgkmcnt(0)"] if cfg.bf16 else
           weight_exponents(cfg, s) + ["s_waitcnt lgkmcnt(0)",
                                       f"v_lshrrev_b32_e32 v{cfg.v_sae + 2}, 23, v{cfg.v_sae + 2}"])
    pf = prefetch_items(cfg, 1) if cfg.xpf else []  # the next unit's block 1 copies, one per matrix instruction
    for j in range(rbe):
        b = cfg.bufid(j)
        nxt = j + 1 < rbe
        bn = cfg.bufid(j + 1)
        place = [[] for _ in range(4)]
        for q in range(4):
            place[q] += [ins for it in pf[4 * j + q:4 * j + q + 1] for ins in it]
        if nxt:
            if j >= 2:  # row tile j - 2's 12 staging operations may be in flight
                place[0].append("s_waitcnt lgkmcnt(10)")
            place[0] += frag_reads(cfg, s, bn, j + 1)
            if not cfg.bf16:
                place[0].append(f"ds_read_b32 v{cfg.v_sae + bn}, v{cfg.v_sadr} offset:{512 * (j + 1) + 4 * s}")
        if j == 0:
            place[1] += ep_setup(cfg)
        if j >= 2:  # row tile j - 2 read back (the fragment reads of row tile j + 1 may still be in flight: 4, and
            # for FP8 its row-scale read)
            place[1] += [f"s_waitcnt lgkmcnt({(4 if cfg.bf16 else 5) if nxt else 0})"] + ep_store_full(cfg, j - 2)
        if j >= 1:
            # the accumulators of row tile j - 1 were last written 4 matrix instructions ago; the nops make
            # the required wait states explicit where few other instructions lie between
            place[2] += (["s_nop 15"] if j == 1 else []) + ep_convert(cfg, j - 1, 0)
            place[3] += ep_convert(cfg, j - 1, 1)
        if nxt:
            place[3] += ["s_waitcnt lgkmcnt(0)"] + ([] if cfg.bf16 else
                                                   [f"v_lshrrev_b32_e32 v{cfg.v_sae + bn}, 23, v{cfg.v_sae + bn}"])
        if j >= 1:
            place[3] += ["s_nop 1"] + ep_stage(cfg, j - 1)
        out.append("s_nop 1")
        q = 0
        for kk in range(2):
            for ct in range(2):
                out += mfma(cfg, s, b, j, ct, kk, False)
                out += place[q]
                q += 1
    return out


def swiglu_epilogue(cfg, rbe):
    """After the loop, for units of rbe row tiles of the up-projection with SwiGLU: the unit's 128 gate
    columns are computed by waves 0 and 1 and the matching 128 up columns by waves 2 and 3, so the pairs meet
    in LDS.  Once every wave is done with the ring (barrier), each row tile's accumulators are rounded to
    bf16 (as the GEMM's output) and written over the ring: row m at m * 512 (gate values 0 .. 127, then up
    values 0 .. 127), 16-byte chunk c (values 8 c .. 8 c + 7 of the row) at position c ^ (m & 31).  %[epb] is
    the address of this lane's 8 bytes in chunk 8 w of its row (the chunk of column tile ct and register
    group g is 8 w + 4 ct + g, an XOR away); row tiles 4 .. 7 use a second set of addresses 64 KB higher, as
    the instruction offset holds 16 bits.  The bf16 pairs alternate between two buffers, so a row tile's
    conversion overlaps the previous row tile's writes.  SwiGLU and the quantisation follow the final
    barrier, in the unit's C++ code."""
    E, E2 = cfg.v_ep, cfg.v_pk  # chunk addresses of row tiles 0 .. 3, and + 64 KB for row tiles 4 .. 7
    out = [f"{700 + rbe}:", "s_waitcnt lgkmcnt(0)", "s_barrier", f"v_mov_b32_e32 v{E}, %[epb]"]
    out += [f"v_xor_b32_e32 v{E + c}, {16 * c}, %[epb]" for c in range(1, 8)]
    if rbe > 4:
        out += [f"v_add_u32_e32 v{E2 + c}, 0x10000, v{E + c}" for c in range(8)]
    out.append("s_nop 15")
    for j in range(rbe):
        T, PK, A = cfg.v_t, cfg.v_rbk + 16 * (j % 2), (E if j < 4 else E2)
        out += [f"v_accvgpr_read_b32 v{T + 16 * ct + r}, a{cfg.acc(j, ct) + r}" for ct in range(2) for r in range(16)]
        out.append("s_nop 1")
        if j:  # row tile j - 2's writes (from this buffer) done, at most 15 LDS operations in flight
            out.append("s_waitcnt lgkmcnt(7)")
        for ct in range(2):
            for g in range(4):
                t, pr = T + 16 * ct + 4 * g, PK + 8 * ct + 2 * g
                out += [f"v_cvt_pk_bf16_f32 v{pr}, v{t}, v{t + 1}", f"v_cvt_pk_bf16_f32 v{pr + 1}, v{t + 2}, v{t + 3}"]
        off = 16384 * (j % 4)
        out += [f"ds_write_b64 v{A + 4 * ct + g}, v[{PK + 8 * ct + 2 * g}:{PK + 8 * ct + 2 * g + 1}]"
                + (f" offset:{off}" if off else "") for ct in range(2) for g in range(4)]
    out += ["s_waitcnt lgkmcnt(0)", "s_branch 7f"]
    return out


def epilogue(cfg, rbe):
    """After the loop, for units of rbe row tiles: store row tile rbe - 2 (staged while the last row tile was
    multiplied) and convert, stage and store row tile rbe - 1, masking rows at or past the unit's end.  A
    wave without columns stores nothing.  The final barrier (label 7, shared) keeps the next unit's copies
    into the ring behind every wave's use of its staging area."""
    if cfg.swiglu:
        return swiglu_epilogue(cfg, rbe)
    out = [f"{700 + rbe}:", "s_cmp_eq_u32 %[won], 0", "s_cbranch_scc1 7f", "s_waitcnt lgkmcnt(0)"]
    out += ep_store_masked(cfg, rbe - 2) + ["s_nop 15", "s_nop 15"]
    out += ep_convert(cfg, rbe - 1, 0) + ep_convert(cfg, rbe - 1, 1) + ["s_nop 1"] + ep_stage(cfg, rbe - 1)
    out += ["s_waitcnt lgkmcnt(0)"] + ep_store_masked(cfg, rbe - 1) + ["s_branch 7f"]
    return out


def prologue(cfg, packed, rbe):
    """The loads of K blocks 0 .. dist - 1, then block 0 in place (the later ones may still be in flight) and
    its row tile 0 read into fragment buffer 2.

    xpf: when bit 0 of %[fl] is set, the previous unit has issued all of this unit's loads of blocks 0 and 1 (its last K
    block the activation copies and the first row-scale group, its end the weights and weight scales into ring
    slots 0 and 1; the offsets already point past them): only the wait for block 0 remains."""
    out = ["s_mov_b32 %[q], 0"]
    for t in range(cfg.dist):
        items, upd = issue_items(cfg, t, packed, rbe)
        out += [ins for it in items for ins in it] + upd
    out += [f"s_waitcnt vmcnt({(cfg.dist - 1) * cfg.ops_for(rbe)})"]
    if cfg.xpf:  # (block 1's weights and weight scale may still be in flight)
        pre = ["s_bitcmp1_b32 %[fl], 0", f"s_cbranch_scc0 {800 + rbe}f", f"s_mov_b32 %[q], {cfg.dist}",
               f"s_waitcnt vmcnt({cfg.ops_for(0)})", f"s_branch {850 + rbe}f", f"{800 + rbe}:"]
        out = pre + out + [f"{850 + rbe}:"]
    out += ["s_barrier"] + frag_reads(cfg, 0, 2, 0) + (
        [] if cfg.bf16 else [f"ds_read_b32 v{cfg.v_sae + 2}, v{cfg.v_sadr}"])
    return out


def program(cfg, packed):
    S = cfg.S
    out = []
    for kk in range(2):
        for p in range(2):
            out.append(f"v_mov_b32_e32 v{cfg.v_aadr + 2 * kk + p}, %[a{kk}{p}]")
    if not cfg.bf16:
        out.append(f"v_mov_b32_e32 v{cfg.v_sadr}, %[sadr]")
    for s in range(1, S):
        for kk in range(2):
            for p in range(2):
                out.append(f"v_add_u32_e32 v{cfg.v_aadr + 4 * s + 2 * kk + p}, {s * cfg.slot}, %[a{kk}{p}]")
    # one prologue and loop body per row-tile count (2 .. rt): no branch between the matrix instructions of a
    # step, and a unit copies the activation rows of its row tiles only
    for r in range(2, cfg.rt):
        out += [f"s_cmp_eq_u32 %[rbe], {r}", f"s_cbranch_scc1 {100 + r}f"]
    for r in range(cfg.rt, 1, -1):
        out += [f"{100 + r}:"] + prologue(cfg, packed, r) + body(cfg, packed, r)
    for r in range(cfg.rt, 1, -1):
        out += epilogue(cfg, r)
    out += ["7:", "s_barrier"]
    if cfg.xpf:
        out += next_unit_weights(cfg, packed)
    return out


def next_unit_weights(cfg, packed):
    """After the unit's final barrier (no wave uses the ring registers any more): the next unit's weights and
    weight scales of K blocks 0 and 1 into ring slots 0 and 1, left in flight for the next unit's loop (the
    code between two loops references none of the loop's registers; a build test checks the compiled kernel).
    The last unit of the workgroup (bit 1 of %[fl] clear) instead waits until nothing is in flight, LDS copies
    included."""
    out = ["s_bitcmp1_b32 %[fl], 1", "s_cbranch_scc0 8f"]
    for t in range(2):
        items, _ = issue_items(cfg, t, packed, 0)
        for it in items:
            for ins in it:
                if ins.startswith("global_load_dwordx4 v["):
                    out.append(ins.replace("%[wo", "%[nwo").replace("%[wb]", "%[nwb]"))
                elif ins.startswith("global_load_dword v"):
                    out.append(ins.replace("%[wso], %[swb]", "%[nwso], %[nswb]") + (" offset:4" if t else ""))
        if t == 0:
            out += [f"v_add_u32_e32 %[nwo{ct}], %[wstep], %[nwo{ct}]" for ct in range(2)]
    return out + ["s_branch 9f", "8:", "s_waitcnt vmcnt(0)", "9:"]


def clobbers(cfg):
    top = cfg.nacc + (0 if cfg.frag_v else 16 * NBUF)
    regs = [f'"v{r}"' for r in range(cfg.v_alo, 256)] + [f'"a{r}"' for r in range(0, top)]
    return ", ".join(regs)


# The 192-row tiles serve experts of about one chunk (each weight byte read by one unit): their weight loads are
# nontemporal.  The 256-row tiles serve experts of many chunks, whose units re-read the weights from L2.
CONFIGS = [Cfg(192, 4, "TALL192", wnt=True, xpf=True), Cfg(256, 4, "TALL256", xpf=True),
           Cfg(192, 4, "SWIGLU_TALL192", wnt=True, swiglu=True), Cfg(256, 4, "SWIGLU_TALL256", swiglu=True),
           Cfg(192, 4, "BF16_TALL192", "bf16", wnt=True), Cfg(256, 4, "BF16_TALL256", "bf16"),
           Cfg(192, 4, "FP4_TALL192", "fp4", wnt=True), Cfg(256, 4, "FP4_TALL256", "fp4")]


def main():
    with open(sys.argv[1], "w") as f:
        f.write("// Generated by gen_fp8_asm.py -- do not edit.\n")
        f.write(f"#define MOE_FP8_TALL_SCALE_ROWS {SCALE_ROWS}\n#define MOE_FP8_TALL_SCALE_GROUP {GROUP}\n")
        for cfg in CONFIGS:
            n = cfg.name if cfg.bf16 or cfg.fp4 or cfg.swiglu else "FP8_" + cfg.name
            f.write(f"// {n}: {cfg.rows} rows, ring {cfg.S}, {cfg.rt} row tiles, {cfg.ops} loads/K block "
                    + ("\n" if cfg.bf16 else "(+1 per scale group)\n"))
            f.write(f"#define MOE_{n}_SLOT_A {cfg.slot_a}\n#define MOE_{n}_SLOT {cfg.slot}\n"
                    f"#define MOE_{n}_SC_OFF {cfg.sc_off}\n#define MOE_{n}_LDS {cfg.lds}\n"
                    f"#define MOE_{n}_APW {cfg.apw}\n#define MOE_{n}_S {cfg.S}\n")
            f.write(f"#define MOE_{n}_AO_OUTS " + ", ".join(f'[ao{i}] "+v"(ao[{i}])' for i in range(cfg.apw))
                    + "\n")

            for suffix, packed in ((("_PACKED", True),) if cfg.fp4 else (("", False), ("_PACKED", True))):
                f.write(f"#define MOE_{n}_LOOP{suffix} \\\n")
                for ln in program(cfg, packed):
                    f.write(f'  "{ln}\\n" \\\n')
                f.write("  \"\"\n")
            f.write(f"#define MOE_{n}_CLOBBERS {clobbers(cfg)}\n")


if __name__ == "__main__":
    main()
