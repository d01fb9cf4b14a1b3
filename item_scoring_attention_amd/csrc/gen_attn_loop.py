"""Generate attn_loop.inc: the key-tile loop of the bf16 MIS attention kernel
as one gfx950 inline-assembly block.

Run ``python gen_attn_loop.py`` in this directory after editing; the output
is committed and the build does not run this script (a CPU test checks that
the committed file matches what this script writes).

What the block computes (one wave = 64 query rows of one head, or 32 in the
QB1 variant; the caller has set up everything the loop needs):

  for each 64-key tile of the visit list (two 32-key sub-tiles each):
    S^T = K Q^T on v_mfma_f32_32x32x16_bf16, Eq. 4 mask on the tiles that
    need it, P = exp2(c S - m) rounded to bf16, row sums, O^T += V^T P^T.

The sub-tiles are software-pipelined: the step of sub-tile j issues the QK
MFMAs of sub-tile j+1 and the PV MFMAs of sub-tile j-1 while the VALU turns
S(j) into P(j), so the matrix cores and the vector ALU work side by side
inside one wave. The running maximum m of a row is only raised when a
sub-tile's largest P exceeds 2^24 (the first visited sub-tile always does,
because m starts at -1e30): then the exact maximum of the sub-tile is taken,
O and the row sum are rescaled (not on the query tile's first sub-tile,
where both are still zero) and P is recomputed.
Any m that was ever a real maximum keeps the result exact, because O and the
row sum are scaled by the same exp2(-m).

The ring's first loads (K(0), K(1), V(0), and with three stages K(2), V(1))
are a second, small block (MIS_ATTN_PROLOGUE_TEXT_*): the kernel issues it
right after its own loads of Q, tile classes and position ids, so all of them
take one round trip, and the loop block starts with them landed.

Register map of the 64-row variant (physical, clobbered by the block;
set_layout gives both variants' maps):
  v[0:31]    S_A   (S^T of a sub-tile, 2 query blocks x 16 fp32)
  v[32:63]   S_B
  v[64:79]   P_A   (P^T bf16, [qb][ks] 4 dwords each)
  v[80:95]   P_B
  then the K and V^T fragment rings (RING x 4 each), exp temporaries,
  mask / rescale temporaries, m, the overflow-check maxima and the
  row-sum selection operand
  a[0:127]   O^T accumulators [qb][db] (operands, pinned)
  a[128:191] Q^T fragments [qb][dstep] (operands, pinned)
  a[192:199] row sums [qb], 4 each: on the matrix cores, so they add exactly
             the bf16 P that O^T += V^T P^T uses. One v_mfma_f32_16x16x32_bf16
             per 16-key quad of P^T: read as its B operand, lane l's 8 values
             are column l % 16, k-group l / 16 (lanes ql and ql + 32 of query
             ql land in k-groups of equal parity, parity ql / 16). The A
             operand selects k-groups of parity (m / 4) % 2 for output row m,
             and lane l holds rows 4 (l / 16) .. +3: so all four accumulator
             registers of lane l hold the sum of the lane's own query ql
             (half the matrix-pipe time of 1^T P^T on a 32 x 32 MFMA, with
             the same per-lane rescale)
"""
from __future__ import annotations

import os

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "attn_loop.inc")

# LDS layout: STAGES K stages of 16 KB from the kernel's LDS base, then
# STAGES V stages. K reads address the K region (ka registers), V reads the V
# region (va registers already point at its start), so DS offsets stay below
# 64 KB. The LDS-direct loads address both through M0.
STAGE_BYTES = 16384
HALF = 8192  # second 32-key half of a 64-key tile


def k_off(stage):
    return STAGE_BYTES * stage


def v_off(stage):
    return STAGE_BYTES * stage


def v_lds(stage, stages):
    return STAGE_BYTES * (stages + stage)

ILV = False


def set_layout(qb: int):
    """Register map for QB query blocks of 32 rows per wave (2: 64 rows, the
    map in the module docstring; 1: 32 rows, small enough for two waves per
    SIMD: S 0-31, P 32-47, 3-deep rings from 48, 8 exp temporaries that the
    rescale path reuses; O^T a[0:63], Q^T a[64:95], row sums a[96:99])."""
    global QB, RING, S_A, S_B, P_A, P_B, KB, VB, E0, NPT, X0, VM, VMX, VNINF, ONES, NUM_V, QA, LS
    QB = qb
    RING = 4 if qb == 2 else 3         # K and V^T fragments in flight (each ring slot is 4 VGPRs)
    S_A, S_B = 0, 16 * qb              # S^T of a sub-tile: 16 fp32 per query block
    P_A, P_B = 32 * qb, 40 * qb        # P^T bf16: 8 dwords per query block
    r0 = 48 * qb                       # start of the fragment rings
    KB = tuple(r0 + 4 * i for i in range(RING))
    VB = tuple(r0 + 4 * RING + 4 * i for i in range(RING))
    E0 = r0 + 8 * RING                 # exp temporaries: NPT pairs in flight
    NPT = 8 if qb == 2 else 4
    # 8 mask / rescale temporaries; with one query block they alias the exp
    # temporaries (the rescale finishes before its softmax starts)
    X0 = E0 + 2 * NPT if qb == 2 else E0
    rest = X0 + 8
    VM = (rest, rest + 1)              # running maxima m (exp2 domain)
    VMX = (rest + 2, rest + 3)         # largest P of the current sub-tile (overflow check)
    VNINF = rest + 4                   # -inf
    ONES = rest + 8                    # 4 VGPRs of bf16 0/1 (lane pattern): A operand of the row-sum MFMAs
    NUM_V = rest + 12
    QA = 64 * qb                       # Q^T fragments a[QA:QA + 32 qb]
    LS = 96 * qb                       # row-sum accumulators [qb], 4 AGPRs each


set_layout(2)

# SGPRs used inside the block
S_T = 40      # visit index of the current tile pair (even)
S_KT = 41     # key tile of the tile being masked
S_TMP = 42    # scalar temporaries s42..s47
S_RSRC = 48   # buffer descriptor s[48:51]
S_LIM = 52
S_SK = 54
S_KEY0 = 55
S_M2 = 56     # s[56:57] compare mask
S_M3 = 58     # s[58:59]
S_OFF = 61
S_NV1 = 62    # scratch
S_LAST = 63
S_VRSRC = 64  # V buffer descriptor s[64:67]
SGPRS = list(range(40, 72))

MFMA = "v_mfma_f32_32x32x16_bf16"
MFMA_RS = "v_mfma_f32_16x16x32_bf16"  # row sums (half the cycles of MFMA)
# VALU cycles placed after each MFMA (one v_mfma_f32_32x32x16_bf16 keeps the
# matrix pipe busy for 32 cycles; an exp costs about 10 issue cycles, other
# VALU 4) and before the first one (while the first K fragment arrives).
SLOT_BUDGET = 24
HEAD_BUDGET = 16
EXP_COST = 10  # issue cycles charged for a v_exp_f32 in that budget


def vr(a, n=1):
    return f"v{a}" if n == 1 else f"v[{a}:{a + n - 1}]"


def ar(a, n=1):
    return f"a{a}" if n == 1 else f"a[{a}:{a + n - 1}]"


def sr(a, n=1):
    return f"s{a}" if n == 1 else f"s[{a}:{a + n - 1}]"


class Block:
    def __init__(self):
        self.lines: list[str] = []
        self.ds: list[str] = []  # tags of DS operations in issue order
        self.done = 0  # number of DS ops known complete

    def emit(self, s: str):
        self.lines.append(s)

    def ds_op(self, tag: str, text: str):
        self.emit(text)
        self.ds.append(tag)

    def wait_ds(self, tag: str):
        """Wait until the last DS op tagged `tag` has completed (in-order completion)."""
        idx = max(i for i, t in enumerate(self.ds) if t == tag)
        if idx < self.done:
            return
        # lgkmcnt(n) leaves at most n operations in flight; with more than 15
        # issued after the target, waiting for 15 still covers the target
        n = min(len(self.ds) - idx - 1, 15)
        self.emit(f"s_waitcnt lgkmcnt({n})")
        self.done = len(self.ds) - n

    def reset_ds(self):
        self.ds = []
        self.done = 0


def softmax_graph(s_cur: int, p_cur: int, c: str):
    """VALU work turning S_cur into P_cur (bf16) and the largest P per row, as
    (text, cost, deps) nodes. Pair i (qb = i // 8, elements 2pi, 2pi+1):
    two FMAs (c s - m), two exps, a convert into dword pi of P_cur[qb] and a
    max3 into VMX[qb]. Pair i uses exp temporaries E0 + 2 (i % NPT), so
    pair i + NPT waits for pair i's convert and max (write after read). The row
    sums are not formed here: they run on the matrix cores."""
    nodes = []

    def add(text, cost, deps):
        nodes.append((text, cost, tuple(deps)))
        return len(nodes) - 1

    last_max = {0: None, 1: None}
    done_pair = {}
    for i in range(8 * QB):
        qb, pi = divmod(i, 8)
        ea = E0 + 2 * (i % NPT)
        eb = ea + 1
        sa = s_cur + 16 * qb + 2 * pi
        m = VM[qb]
        war = done_pair.get(i - NPT, ())
        fa = add(f"v_fma_f32 {vr(ea)}, {vr(sa)}, {c}, -{vr(m)}", 4, war)
        fb = add(f"v_fma_f32 {vr(eb)}, {vr(sa + 1)}, {c}, -{vr(m)}", 4, war)
        xa = add(f"v_exp_f32 {vr(ea)}, {vr(ea)}", EXP_COST, [fa])
        xb = add(f"v_exp_f32 {vr(eb)}, {vr(eb)}", EXP_COST, [fb])
        cv = add(f"v_cvt_pk_bf16_f32 {vr(p_cur + 8 * qb + pi)}, {vr(ea)}, {vr(eb)}", 4, [xa, xb])
        lm = last_max[qb]
        mx = add(f"v_max_f32 {vr(VMX[qb])}, {vr(ea)}, {vr(eb)}" if lm is None else
                 f"v_max3_f32 {vr(VMX[qb])}, {vr(VMX[qb])}, {vr(ea)}, {vr(eb)}", 4,
                 [xa, xb] + ([] if lm is None else [lm]))
        last_max[qb] = mx
        done_pair[i] = (cv, mx)
    return nodes


def softmax_ops(s_cur: int, p_cur: int, c: str) -> list[str]:
    """The softmax work in a plain order for the slow path: nodes in creation
    order, with one independent instruction (or a nop) after every exp."""
    ops = []
    for text, _, deps in softmax_graph(s_cur, p_cur, c):
        if ops and ops[-1].startswith("v_exp_f32") and text.split()[0] != "v_exp_f32":
            ops.append("s_nop 1")
        ops.append(text)
    return ops


def schedule(nodes, slots: int, budget: int, head_budget: int):
    """Place every node in one of slots + 1 groups (group 0 runs before the
    first MFMA, group k after MFMA k - 1) so that a node lands in a later
    group than each node it depends on (at least one MFMA between producer
    and consumer, which covers the exp latency and the trans-use hazard) and
    no group exceeds its cycle budget when it can be helped."""
    group = [0] * len(nodes)
    load = [0] * (slots + 1)
    out = [[] for _ in range(slots + 1)]
    for n, (text, cost, deps) in enumerate(nodes):
        g = max((group[d] + 1 for d in deps), default=0)
        cap = lambda k: head_budget if k == 0 else budget
        while g < slots and load[g] + cost > cap(g):
            g += 1
        g = min(g, slots)
        # a consumer in its producer's group would lose the MFMA between them
        # (exp latency and the transcendental-use hazard): refuse the budget
        if any(group[d] >= g for d in deps):
            raise ValueError(f"VALU budget {budget} leaves no MFMA between {text!r} and its producer")
        group[n] = g
        load[g] += cost
        out[g].append(text)
    return out


def k_read(b: Block, ds: int, koff: int, tag: str):
    b.ds_op(tag, f"ds_read_b128 {vr(KB[ds % RING], 4)}, %[ka{ds}] offset:{koff}")


def v_read(b: Block, f: int, voff: int, tag: str):
    ks, db = divmod(f, 4)
    buf = VB[f % RING]
    off = voff + 4096 * ks
    b.ds_op(tag, f"ds_read_b64_tr_b16 {vr(buf, 2)}, %[va{db}] offset:{off}")
    b.ds_op(tag, f"ds_read_b64_tr_b16 {vr(buf + 2, 2)}, %[va{db}] offset:{off + 2048}")


def hoist_first_reads(b: Block, koff: int, voff: int):
    """The first RING K and V fragment reads of a step, issued ahead of it
    (tagged N..., picked up by the step as its own)."""
    for ds in range(RING):
        k_read(b, ds, koff, f"Nk{ds}")
    for f in range(RING):
        v_read(b, f, voff, f"Nv{f}")


def step(b: Block, s_cur, s_next, p_cur, p_prev, koff, voff, c, side=(), pre=False, nxt=None):
    """One pipelined sub-tile: QK(next) + PV(prev) MFMAs interleaved with softmax(cur).

    `side` holds small instruction groups (descriptor set-up and the next
    tiles' LDS-direct loads) issued one after each MFMA from the second on,
    so their issue cost hides under the matrix pipe. `pre`: the step's first
    RING K and V fragment reads were issued ahead of it (by the previous step
    or the block's start). `nxt` = (koff, voff) of the next step: its first
    RING fragments are read here as soon as their ring slots are free, so
    the next step's first MFMA does not wait for a read issued at its start."""
    if pre:
        # the fragments read ahead are all this step tracks; everything
        # issued before them has completed (LDS reads complete in order)
        b.ds = [t[1:] for t in b.ds if t.startswith("N")]
        b.done = 0
    else:
        b.reset_ds()
    side = list(side)
    valu = schedule(softmax_graph(s_cur, p_cur, c), 16 * QB, SLOT_BUDGET, HEAD_BUDGET)
    vi = 0

    def valu_group():
        nonlocal vi
        if vi < len(valu):
            for ln in valu[vi]:
                b.emit(ln)
            vi += 1

    if not pre:
        for ds in range(RING):
            k_read(b, ds, koff, f"k{ds}")
        for f in range(RING):
            v_read(b, f, voff, f"v{f}")
    valu_group()
    # MFMA order: all QK then all PV, or (ILV) alternating, so that the QK
    # accumulation chain of a single query block never runs back to back
    order = ([("qk", i) for i in range(8 * QB)] + [("pv", i) for i in range(8 * QB)] if not ILV else
             [(kind, i) for i in range(8 * QB) for kind in ("qk", "pv")])
    for slot, (kind, idx) in enumerate(order):
        if kind == "qk":
            ds, qb = divmod(idx, QB)
            b.wait_ds(f"k{ds}")
            acc = vr(s_next + 16 * qb, 16)
            src_c = "0" if ds == 0 else acc
            b.emit(f"{MFMA} {acc}, {vr(KB[ds % RING], 4)}, {ar(QA + 32 * qb + 4 * ds, 4)}, {src_c}")
            if qb == QB - 1 and ds + RING < 8:
                k_read(b, ds + RING, koff, f"k{ds + RING}")
            elif qb == QB - 1 and nxt:  # last use of this ring slot: the next step's fragment
                k_read(b, ds % RING, nxt[0], f"Nk{ds % RING}")
        else:
            f, qb = divmod(idx, QB)
            ks, db = divmod(f, 4)
            b.wait_ds(f"v{f}")
            o = ar(16 * (4 * qb + db), 16)
            b.emit(f"{MFMA} {o}, {vr(VB[f % RING], 4)}, {vr(p_prev + 8 * qb + 4 * ks, 4)}, {o}")
            if qb == QB - 1 and f + RING < 8:
                v_read(b, f + RING, voff, f"v{f + RING}")
            elif qb == QB - 1 and nxt:
                v_read(b, f % RING, nxt[1], f"Nv{f % RING}")
            if qb == QB - 1 and db == 3:
                for q in range(QB):
                    ls = ar(LS + 4 * q, 4)
                    b.emit(f"{MFMA_RS} {ls}, {vr(ONES, 4)}, {vr(p_prev + 8 * q + 4 * ks, 4)}, {ls}")
        if slot >= 1 and side:
            for ln in side.pop(0):
                b.emit(ln)
        valu_group()
    for g in side:
        for ln in g:
            b.emit(ln)
    while vi < len(valu):
        valu_group()


def mask_code(b: Block, s_cur: int, half: int, skip_label: str):
    """Eq. 4 mask of S_cur (sub-tile `half` of key tile S_KT) when the visit needs it."""
    # visible iff key <= jt and (key < lq or key >= jb); key = key0 + 8(a/4) + a%4 + 4g
    b.emit(f"s_lshl_b32 {sr(S_KEY0)}, {sr(S_KT)}, 6")
    if half:
        b.emit(f"s_add_u32 {sr(S_KEY0)}, {sr(S_KEY0)}, 32")
    for a in range(16):
        ka = 8 * (a // 4) + a % 4
        b.emit(f"s_add_u32 {sr(S_SK)}, {sr(S_KEY0)}, {ka}")
        for qb in range(QB):
            b.emit(f"v_cmp_le_i32 {sr(S_M2, 2)}, {sr(S_SK)}, %[rjt{qb}]")
            b.emit(f"v_cmp_lt_i32 {sr(S_M3, 2)}, {sr(S_SK)}, %[rlq]")
            b.emit(f"v_cmp_ge_i32 vcc, {sr(S_SK)}, %[rjb{qb}]")
            b.emit(f"s_or_b64 vcc, vcc, {sr(S_M3, 2)}")
            b.emit(f"s_and_b64 vcc, vcc, {sr(S_M2, 2)}")
            x = s_cur + 16 * qb + a
            b.emit(f"v_cndmask_b32 {vr(x)}, {vr(VNINF)}, {vr(x)}, vcc")
    b.emit(f"{skip_label}:")


def slow_path(b: Block, s_cur, p_cur, c, label, ret, first=False):
    """Raise m to the sub-tile maximum, rescale O and the row sums, recompute P.

    `first`: this step can hold the query tile's first sub-tile (visit 0's
    first half). There O and the row sums are still zero (the PV and row-sum
    MFMAs so far multiplied zero P), so on visit 0 the rescale is skipped."""
    b.emit(f"{label}:")
    b.emit("s_nop 7")
    b.emit("s_nop 7")
    b.emit("s_nop 7")
    for qb in range(QB):
        s0 = s_cur + 16 * qb
        x, y, z, al = X0, X0 + 1, X0 + 2, X0 + 3
        b.emit(f"v_max3_f32 {vr(x)}, {vr(s0)}, {vr(s0 + 1)}, {vr(s0 + 2)}")
        for a in range(3, 15, 2):
            b.emit(f"v_max3_f32 {vr(x)}, {vr(x)}, {vr(s0 + a)}, {vr(s0 + a + 1)}")
        b.emit(f"v_max_f32 {vr(x)}, {vr(x)}, {vr(s0 + 15)}")
        b.emit(f"v_mov_b32 {vr(y)}, {vr(x)}")
        b.emit(f"v_mov_b32 {vr(z)}, {vr(x)}")
        b.emit("s_nop 1")
        b.emit(f"v_permlane32_swap_b32 {vr(y)}, {vr(z)}")
        b.emit("s_nop 1")
        b.emit(f"v_max3_f32 {vr(x)}, {vr(x)}, {vr(y)}, {vr(z)}")
        b.emit(f"v_mul_f32 {vr(x)}, {c}, {vr(x)}")
        b.emit(f"v_max_f32 {vr(x)}, {vr(x)}, {vr(VM[qb])}")
        b.emit(f"v_sub_f32 {vr(al)}, {vr(VM[qb])}, {vr(x)}")
        b.emit(f"v_exp_f32 {vr(al)}, {vr(al)}")
        b.emit(f"v_mov_b32 {vr(VM[qb])}, {vr(x)}")
        if first:
            b.emit(f"s_cmp_eq_u32 {sr(S_T)}, 0")
            b.emit(f"s_cbranch_scc1 {label}_nr{qb}")
        tmps = [X0 + 4, X0 + 5, X0 + 6, X0 + 7]
        for i, acc in enumerate(list(range(64 * qb, 64 * qb + 64)) + list(range(LS + 4 * qb, LS + 4 * qb + 4))):
            t = tmps[i % 4]
            b.emit(f"v_accvgpr_read_b32 {vr(t)}, {ar(acc)}")
            b.emit(f"v_mul_f32 {vr(t)}, {vr(t)}, {vr(al)}")
            b.emit(f"v_accvgpr_write_b32 {ar(acc)}, {vr(t)}")
        if first:
            b.emit(f"{label}_nr{qb}:")
    for ln in softmax_ops(s_cur, p_cur, c):
        b.emit(ln)
    b.emit(f"s_branch {ret}")


def tile_of(b: Block, dst: int, idx_reg: str):
    """dst = idx < a_end ? idx : b_start + idx - a_end."""
    b.emit(f"s_sub_u32 {sr(S_TMP)}, {idx_reg}, %[a_end]")
    b.emit(f"s_add_u32 {sr(S_TMP)}, {sr(S_TMP)}, %[b_start]")
    b.emit(f"s_cmp_lt_u32 {idx_reg}, %[a_end]")
    b.emit(f"s_cselect_b32 {sr(dst)}, {idx_reg}, {sr(S_TMP)}")


def dma_setup(b: Block, vis_add: int, is_k: bool, rsrc: int):
    """Buffer descriptor of visit S_T + vis_add: K or V rows of its key tile up
    to the request end; a zero range when the visit does not exist (the loads
    then touch no memory and write nothing)."""
    for ln in dma_setup_lines(vis_add, is_k, rsrc):
        b.emit(ln)


def dma_setup_lines(vis_add: int, is_k: bool, rsrc: int) -> list[str]:
    base_lo, base_hi = ("%[kb_lo]", "%[kb_hi]") if is_k else ("%[vb_lo]", "%[vb_hi]")
    t = Block()
    t.emit(f"s_add_u32 {sr(S_NV1)}, {sr(S_T)}, {vis_add}")
    tile_of(t, S_LAST, sr(S_NV1))
    t.emit(f"s_mul_i32 {sr(S_OFF)}, {sr(S_LAST)}, %[rb64]")
    t.emit(f"s_add_u32 {sr(rsrc)}, {base_lo}, {sr(S_OFF)}")
    t.emit(f"s_addc_u32 {sr(rsrc + 1)}, {base_hi}, 0")
    t.emit(f"s_sub_u32 {sr(rsrc + 2)}, %[nrec], {sr(S_OFF)}")
    t.emit(f"s_cmp_lt_u32 {sr(S_NV1)}, %[nvis]")
    t.emit(f"s_cselect_b32 {sr(rsrc + 2)}, {sr(rsrc + 2)}, 0")
    t.emit(f"s_mov_b32 {sr(rsrc + 3)}, 0x20000")
    return t.lines


# scalar instructions of descriptor set-up placed after one MFMA
SETUP_CHUNK = 4


def dma_groups(is_k: bool, rsrc: int, lds_byte: int, dpw: int) -> list[list[str]]:
    """The LDS-direct loads of one tile (this wave's rows), one group per load.

    Load i's per-lane VGPR offset (ko{i} / vo{i}) holds the whole byte offset
    of the lane's chunk inside the tile, wave row and row group included, and
    the SGPR offset is 0: the buffer range check covers the VGPR offset (plus
    the instruction offset) but not the SGPR offset, so rows past the
    request's end must show in the VGPR offset to read as nothing."""
    groups = []
    for i in range(dpw):
        g = [f"s_add_u32 m0, %[wlds], {lds_byte + 1024 * i}"]
        voff = f"%[ko{i}]" if is_k else f"%[vo{i}]"
        g.append(f"buffer_load_dwordx4 {voff}, {sr(rsrc, 4)}, 0 offen lds")
        groups.append(g)
    return groups


def barrier_dma(b: Block, tp: int, dpw: int, stages: int) -> list[list[str]]:
    """At tile t' = S_T + tp: wait for the loads tile t' still needs, barrier
    (every wave is done with K(t') and V(t'-1)); the returned side groups set
    up and issue the loads of K(t' + STAGES) into K stage tp and
    V(t' + STAGES - 1) into V stage tp - 1 during the next step. Every
    barrier issues the same 2 dpw loads, so the loads still allowed in flight
    are a constant: those of the last STAGES - 2 barriers, or with four
    stages or more of the last STAGES - 3 (the steps then read K(t' + 1) and
    V(t') before barrier t', so they must be complete by barrier t' - 1:
    issued at barrier t' - 3, two visits earlier, as with three stages)."""
    in_flight = stages - 3 if stages >= 4 else stages - 2
    b.emit(f"s_waitcnt vmcnt({2 * dpw * in_flight})")
    b.emit("s_barrier")

    def chunks(lines):
        return [lines[i:i + SETUP_CHUNK] for i in range(0, len(lines), SETUP_CHUNK)]

    return (chunks(dma_setup_lines(tp + stages, True, S_RSRC)) + dma_groups(True, S_RSRC, k_off(tp), dpw) +
            chunks(dma_setup_lines(tp + stages - 1, False, S_VRSRC)) +
            dma_groups(False, S_VRSRC, v_lds((tp - 1) % stages, stages), dpw))


def pv_tail(b: Block, p_prev: int, voff: int):
    b.reset_ds()
    for f in range(8):
        ks, db = divmod(f, 4)
        buf = VB[f % RING]
        off = voff + 4096 * ks
        b.ds_op(f"v{f}", f"ds_read_b64_tr_b16 {vr(buf, 2)}, %[va{db}] offset:{off}")
        b.ds_op(f"v{f}", f"ds_read_b64_tr_b16 {vr(buf + 2, 2)}, %[va{db}] offset:{off + 2048}")
        if f >= 2:
            g = f - 2
            gks, gdb = divmod(g, 4)
            b.wait_ds(f"v{g}")
            for qb in range(QB):
                o = ar(16 * (4 * qb + gdb), 16)
                b.emit(f"{MFMA} {o}, {vr(VB[g % RING], 4)}, {vr(p_prev + 8 * qb + 4 * gks, 4)}, {o}")
    for g in (6, 7):
        gks, gdb = divmod(g, 4)
        b.wait_ds(f"v{g}")
        for qb in range(QB):
            o = ar(16 * (4 * qb + gdb), 16)
            b.emit(f"{MFMA} {o}, {vr(VB[g % RING], 4)}, {vr(p_prev + 8 * qb + 4 * gks, 4)}, {o}")
    for ks in range(2):
        for q in range(QB):
            ls = ar(LS + 4 * q, 4)
            b.emit(f"{MFMA_RS} {ls}, {vr(ONES, 4)}, {vr(p_prev + 8 * q + 4 * ks, 4)}, {ls}")


def loop_block(dpw: int, stages: int) -> list[str]:
    b = Block()
    c = "%[c]"
    b.emit("s_waitcnt vmcnt(0) lgkmcnt(0)")
    # ---- init
    for i in range(64 * QB):
        b.emit(f"v_accvgpr_write_b32 {ar(i)}, 0")
    for i in range(8 * QB):
        b.emit(f"v_mov_b32 {vr(P_B + i)}, 0")
    for i in range(4 * QB):
        b.emit(f"v_accvgpr_write_b32 {ar(LS + i)}, 0")
    for qb in range(QB):
        b.emit(f"v_mov_b32 {vr(VM[qb])}, 0xf149f2ca")  # -1e30
    for i in range(4):
        b.emit(f"v_mov_b32 {vr(ONES + i)}, %[sel]")  # bf16 (1, 1) or (0, 0) by lane
    b.emit(f"v_mov_b32 {vr(VNINF)}, 0xff800000")
    b.emit(f"s_mov_b32 {sr(S_LIM)}, 0x4b800000")  # 2^24
    b.emit(f"s_mov_b32 {sr(S_T)}, 0")
    # ---- the prologue loads (prologue_block) have landed: the block's first
    # wait covers them. Every wave's share of K(0) is in LDS after the barrier.
    b.emit("s_barrier")
    b.reset_ds()
    for ds in range(8):
        b.ds_op(f"k{ds}", f"ds_read_b128 {vr(KB[ds % RING], 4)}, %[ka{ds}] offset:{k_off(0)}")
        if ds >= 2:
            g = ds - 2
            b.wait_ds(f"k{g}")
            for qb in range(QB):
                acc = vr(S_A + 16 * qb, 16)
                b.emit(f"{MFMA} {acc}, {vr(KB[g % RING], 4)}, {ar(QA + 32 * qb + 4 * g, 4)}, "
                       f"{'0' if g == 0 else acc}")
    for g in (6, 7):
        b.wait_ds(f"k{g}")
        for qb in range(QB):
            acc = vr(S_A + 16 * qb, 16)
            b.emit(f"{MFMA} {acc}, {vr(KB[g % RING], 4)}, {ar(QA + 32 * qb + 4 * g, 4)}, {acc}")
    for _ in range(3):
        b.emit("s_nop 7")
    # the first step's first fragments (its PV reads the zeroed last V stage)
    hoist_first_reads(b, k_off(0) + HALF, v_off(stages - 1) + HALF)
    # ---- main loop over groups of STAGES tiles (S_T a multiple of STAGES at the top)
    b.emit("L_loop:")
    pos = 0
    slow = []
    side = []
    masks = []
    for tp in range(stages):
        # key tile of visit t + tp, and whether its sub-tiles need the mask
        b.emit(f"s_add_u32 {sr(S_NV1)}, {sr(S_T)}, {tp}")
        tile_of(b, S_KT, sr(S_NV1))
        for h in range(2):
            s_cur, s_next = (S_A, S_B) if h == 0 else (S_B, S_A)
            p_cur, p_prev = (P_A, P_B) if h == 0 else (P_B, P_A)
            if h == 0:  # QK: second half of tile t'; PV: second half of tile t' - 1
                koff = k_off(tp) + HALF
                voff = v_off((tp - 1) % stages) + HALF
                # next: QK first half of tile t' + 1, PV first half of tile t'.
                # Read ahead only with four stages: K(t' + 1) and V(t') are then
                # complete and visible from the last barrier on (with fewer
                # stages only after the coming one)
                nxt = (k_off((tp + 1) % stages), v_off(tp)) if stages >= 4 else None
                pre = True
            else:  # QK: first half of tile t' + 1; PV: first half of tile t'
                koff = k_off((tp + 1) % stages)
                voff = v_off(tp)
                # next: tile t' + 1's h = 0 step (no barrier in between)
                nxt = (k_off((tp + 1) % stages) + HALF, v_off(tp) + HALF)
                pre = stages >= 4
            b.emit(f"s_add_u32 {sr(S_NV1)}, {sr(S_T)}, {tp}")
            b.emit(f"s_cmp_ge_u32 {sr(S_NV1)}, %[a_full]")
            b.emit(f"s_cbranch_scc1 L_mask{pos}")
            b.emit(f"L_nomask{pos}:")
            masks.append((s_cur, h, pos))
            step(b, s_cur, s_next, p_cur, p_prev, koff, voff, c, side, pre=pre, nxt=nxt)
            side = []
            b.emit(f"v_cmp_lt_f32 vcc, {sr(S_LIM)}, {vr(VMX[0])}")
            if QB == 2:
                b.emit(f"v_cmp_lt_f32 {sr(S_M2, 2)}, {sr(S_LIM)}, {vr(VMX[1])}")
                b.emit(f"s_or_b64 vcc, vcc, {sr(S_M2, 2)}")
            b.emit(f"s_cbranch_vccnz L_slow{pos}")
            b.emit(f"L_ret{pos}:")
            slow.append((s_cur, p_cur, f"L_slow{pos}", f"L_ret{pos}"))
            if h == 0:
                side = barrier_dma(b, tp, dpw, stages)
            pos += 1
        # leave after the last visited tile: its second half still needs PV
        b.emit(f"s_add_u32 {sr(S_NV1)}, {sr(S_T)}, {tp + 1}")
        b.emit(f"s_cmp_lt_u32 {sr(S_NV1)}, %[nvis]")
        b.emit(f"s_cbranch_scc0 L_exit{tp}")
    b.emit(f"s_add_u32 {sr(S_T)}, {sr(S_T)}, {stages}")
    b.emit("s_branch L_loop")
    for tp in range(stages):
        b.emit(f"L_exit{tp}:")
        pv_tail(b, P_B, v_off(tp) + HALF)
        b.emit("s_branch L_done")
    b.emit("L_done:")
    b.emit("s_waitcnt vmcnt(0)")  # no load may still be writing LDS when the waves end
    for _ in range(3):
        b.emit("s_nop 7")
    b.emit(f"v_accvgpr_read_b32 %[l0], {ar(LS)}")
    if QB == 2:
        b.emit(f"v_accvgpr_read_b32 %[l1], {ar(LS + 4)}")
    b.emit("s_branch L_end")
    for i, args in enumerate(slow):
        slow_path(b, *args[:2], c, *args[2:], first=(i == 0))
    # masks run out of line, so the common path takes no branch
    for s_cur, h, mpos in masks:
        b.emit(f"L_mask{mpos}:")
        mask_code(b, s_cur, h, f"L_mdone{mpos}")
        b.emit(f"s_branch L_nomask{mpos}")
    b.emit("L_end:")
    return [ln for ln in b.lines if ln]


def prologue_order(stages: int) -> list[tuple[int, bool]]:
    """The loads the barriers of visits -STAGES+1 .. -1 would have issued, K(0)
    first: K(0), then K(j), V(j - 1) for j = 1 .. STAGES - 1."""
    out = [(0, True)]
    for j in range(1, stages):
        out += [(j, True), (j - 1, False)]
    return out


def prologue_block(dpw: int, stages: int) -> list[str]:
    """The ring's first loads as a block of their own. The kernel issues it
    right after its own loads (Q, tile classes, position ids) and before it
    uses any of their results, so all of them travel in one round trip; the
    kernel's wait for its own loads then also covers these (loads complete in
    order), and the loop block starts with every prologue load landed."""
    b = Block()
    b.emit(f"s_mov_b32 {sr(S_T)}, 0")
    for v, is_k in prologue_order(stages):
        rsrc = S_RSRC if is_k else S_VRSRC
        dma_setup(b, v, is_k, rsrc)
        lds = k_off(v) if is_k else v_lds(v, stages)
        for g in dma_groups(is_k, rsrc, lds, dpw):
            for ln in g:
                b.emit(ln)
    return [ln for ln in b.lines if ln]


def clobbers() -> list[str]:
    regs = [f'"v{i}"' for i in range(NUM_V)]
    regs += [f'"s{i}"' for i in SGPRS]
    regs += [f'"a{i}"' for i in range(LS, LS + 4 * QB)]
    regs += ['"vcc"', '"scc"', '"m0"', '"memory"']
    return regs


HEADER = """// Generated by gen_attn_loop.py; do not edit by hand.
// The key-tile loop of the bf16 MIS attention kernel as one gfx950 asm block
// (register map and pipeline: see gen_attn_loop.py).
"""


# (macro suffix, LDS-direct loads per wave and tile, K/V stages, query blocks per wave)
VARIANTS = (("DPW4", 4, 4, 2), ("DPW8", 8, 2, 2), ("QB1", 4, 2, 1))


def render() -> str:
    out = [HEADER]
    for name, dpw, stages, qb in VARIANTS:
        set_layout(qb)
        lines = loop_block(dpw, stages)
        # labels must be unique per asm instance: %= expands to a per-instance number
        text = []
        for ln in lines:
            ln = ln.replace("L_", "L%=_")
            text.append(f'  "{ln}\\n"')
        out.append(f"#define MIS_ATTN_LOOP_TEXT_{name} \\")
        out.append(" \\\n".join(text))
        out.append("")
        text = [f'  "{ln}\\n"' for ln in prologue_block(dpw, stages)]
        out.append(f"#define MIS_ATTN_PROLOGUE_TEXT_{name} \\")
        out.append(" \\\n".join(text))
        out.append("")
    set_layout(2)
    out.append("#define MIS_ATTN_LOOP_CLOBBERS " + ", ".join(clobbers()))
    set_layout(1)
    out.append("#define MIS_ATTN_LOOP_CLOBBERS_QB1 " + ", ".join(clobbers()))
    out.append("#define MIS_ATTN_PROLOGUE_CLOBBERS " + ", ".join(
        [f'"s{i}"' for i in SGPRS] + ['"scc"', '"m0"', '"memory"']))
    set_layout(2)
    out.append("")
    return "\n".join(out)


def main():
    with open(OUT, "w") as f:
        f.write(render())


if __name__ == "__main__":
    main()
