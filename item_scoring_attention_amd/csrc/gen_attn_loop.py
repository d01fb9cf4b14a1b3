"""Generate attn_loop.inc: the key-tile loop of the bf16 MIS attention kernel
as one gfx950 inline-assembly block.

Run ``python gen_attn_loop.py`` in this directory after editing; the output
is committed and the build does not run this script (a CPU test checks that
the committed file matches what this script writes).

What the block computes (one wave = 64 query rows of one head; the caller
has set up everything the loop needs):

  for each 64-key tile of the visit list (two 32-key sub-tiles each):
    S^T = K Q^T on v_mfma_f32_32x32x16_bf16, Eq. 4 mask on the tiles that
    need it, P = exp2(c S - m) rounded to bf16, row sums, O^T += V^T P^T.

The sub-tiles are software-pipelined: the step of sub-tile j issues the QK
MFMAs of sub-tile j+1 and the PV MFMAs of sub-tile j-1 while the VALU turns
S(j) into P(j), so the matrix cores and the vector ALU work side by side
inside one wave (one wave per SIMD). The running maximum m of a row is only
raised when a sub-tile's partial row sum exceeds 2^24 (the first visited
sub-tile always does, because m starts at -1e30): then the exact maximum of
the sub-tile is taken, O and the row sum are rescaled and P is recomputed.
Any m that was ever a real maximum keeps the result exact, because O and the
row sum are scaled by the same exp2(-m).

Register map (physical, clobbered by the block):
  v[0:31]    S_A   (S^T of a sub-tile, 2 query blocks x 16 fp32)
  v[32:63]   S_B
  v[64:79]   P_A   (P^T bf16, [qb][ks] 4 dwords each)
  v[80:95]   P_B
  v[96:107]  K fragment ring (3 x 4)
  v[108:119] V^T fragment ring (3 x 4)
  v[120:127] exp temporaries
  v[128:135] mask / rescale temporaries
  v136, v137 running maxima m (exp2 domain), v138, v139 row sums l,
  v140, v141 partial row sums of the current sub-tile (v143, v144 second
             chains), v142 -inf
  a[0:127]   O^T accumulators [qb][db] (operands, pinned)
  a[128:191] Q^T fragments [qb][dstep] (operands, pinned)
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

S_A, S_B, P_A, P_B = 0, 32, 64, 80
KB = (96, 100, 104)
VB = (108, 112, 116)
E0 = 120
X0 = 128
VM = (136, 137)
VL = (138, 139)
VT = (140, 141)
VNINF = 142
VT2 = (143, 144)
NUM_V = 145

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
S_SO = 60     # soffset of a DMA instruction
S_OFF = 61
S_NV1 = 62    # scratch
S_LAST = 63
S_NL = 46     # LDS-direct loads issued at the previous barrier (still allowed in flight)
SGPRS = list(range(40, 64))

MFMA = "v_mfma_f32_32x32x16_bf16"


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
        after = len(self.ds) - idx - 1
        assert after <= 15, "lgkmcnt holds at most 15 outstanding operations"
        self.emit(f"s_waitcnt lgkmcnt({after})")
        self.done = idx + 1

    def reset_ds(self):
        self.ds = []
        self.done = 0


def softmax_ops(s_cur: int, p_cur: int, c: str) -> list[str]:
    """VALU stream turning S_cur into P_cur and the partial row sums VT.

    Pair i (qb = i // 8, elements 2pi, 2pi+1) writes dword pi of P_cur[qb]:
    two FMAs (c s - m), two exps, one convert to bf16, then the two rounded
    values are unpacked (shift, mask) and added to the row-sum chains VT[qb]
    and VT2[qb], so the sums hold exactly the P that the PV product uses.
    (v_dot2_f32_bf16 would add a rounded pair in one instruction, but it does
    not run beside the MFMAs.) The unpack and adds of pair i-1 are placed
    inside pair i, so no instruction reads an exp result it directly follows
    and no chain add waits on the instruction before it."""
    ops = []

    def tail(i):
        qb, pi = divmod(i, 8)
        pd = p_cur + 8 * qb + pi
        ra, rb = X0 + 4 + 2 * (i % 2), X0 + 5 + 2 * (i % 2)
        unpack = [f"v_lshlrev_b32 {vr(ra)}, 16, {vr(pd)}",
                  f"v_and_b32 {vr(rb)}, 0xffff0000, {vr(pd)}"]
        if pi == 0:
            adds = [f"v_mov_b32 {vr(VT[qb])}, {vr(ra)}", f"v_mov_b32 {vr(VT2[qb])}, {vr(rb)}"]
        else:
            adds = [f"v_add_f32 {vr(VT[qb])}, {vr(VT[qb])}, {vr(ra)}",
                    f"v_add_f32 {vr(VT2[qb])}, {vr(VT2[qb])}, {vr(rb)}"]
        return unpack, adds

    for i in range(16):
        qb, pi = divmod(i, 8)
        ea = E0 + 2 * (i % 4)
        eb = ea + 1
        sa = s_cur + 16 * qb + 2 * pi
        m = VM[qb]
        ops += [f"v_fma_f32 {vr(ea)}, {vr(sa)}, {c}, -{vr(m)}",
                f"v_fma_f32 {vr(eb)}, {vr(sa + 1)}, {c}, -{vr(m)}",
                f"v_exp_f32 {vr(ea)}, {vr(ea)}"]
        prev = tail(i - 1) if i else None
        if prev:
            ops += prev[0]
        ops.append(f"v_exp_f32 {vr(eb)}, {vr(eb)}")
        ops += prev[1] if prev else ["s_nop 1"]
        ops.append(f"v_cvt_pk_bf16_f32 {vr(p_cur + 8 * qb + pi)}, {vr(ea)}, {vr(eb)}")
    unpack, adds = tail(15)
    ops += unpack + adds
    ops += [f"v_add_f32 {vr(VT[q])}, {vr(VT[q])}, {vr(VT2[q])}" for q in range(2)]
    return ops


def step(b: Block, s_cur, s_next, p_cur, p_prev, koff, voff, c):
    """One pipelined sub-tile: QK(next) + PV(prev) MFMAs interleaved with softmax(cur)."""
    b.reset_ds()
    flat = softmax_ops(s_cur, p_cur, c)
    head = 6  # VALU issued before the first MFMA (covers the first K read)
    per = -(-(len(flat) - head) // 32)
    valu = [flat[:head]] + [flat[head + per * k: head + per * (k + 1)] for k in range(32)]
    vi = 0

    def k_read(ds):
        b.ds_op(f"k{ds}", f"ds_read_b128 {vr(KB[ds % 3], 4)}, %[ka{ds}] offset:{koff}")

    def v_read(f):
        ks, db = divmod(f, 4)
        buf = VB[f % 3]
        off = voff + 4096 * ks
        b.ds_op(f"v{f}", f"ds_read_b64_tr_b16 {vr(buf, 2)}, %[va{db}] offset:{off}")
        b.ds_op(f"v{f}", f"ds_read_b64_tr_b16 {vr(buf + 2, 2)}, %[va{db}] offset:{off + 2048}")

    def valu_group():
        nonlocal vi
        if vi < len(valu):
            for ln in valu[vi]:
                b.emit(ln)
            vi += 1

    for ds in range(3):
        k_read(ds)
    for f in range(3):
        v_read(f)
    valu_group()
    for slot in range(32):
        if slot < 16:
            ds, qb = divmod(slot, 2)
            b.wait_ds(f"k{ds}")
            acc = vr(s_next + 16 * qb, 16)
            src_c = "0" if ds == 0 else acc
            b.emit(f"{MFMA} {acc}, {vr(KB[ds % 3], 4)}, {ar(128 + 32 * qb + 4 * ds, 4)}, {src_c}")
            if qb == 1 and ds + 3 < 8:
                k_read(ds + 3)
        else:
            f, qb = divmod(slot - 16, 2)
            ks, db = divmod(f, 4)
            b.wait_ds(f"v{f}")
            o = ar(16 * (4 * qb + db), 16)
            b.emit(f"{MFMA} {o}, {vr(VB[f % 3], 4)}, {vr(p_prev + 8 * qb + 4 * ks, 4)}, {o}")
            if qb == 1 and f + 3 < 8:
                v_read(f + 3)
        valu_group()
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
        for qb in range(2):
            b.emit(f"v_cmp_le_i32 {sr(S_M2, 2)}, {sr(S_SK)}, %[rjt{qb}]")
            b.emit(f"v_cmp_lt_i32 {sr(S_M3, 2)}, {sr(S_SK)}, %[rlq]")
            b.emit(f"v_cmp_ge_i32 vcc, {sr(S_SK)}, %[rjb{qb}]")
            b.emit(f"s_or_b64 vcc, vcc, {sr(S_M3, 2)}")
            b.emit(f"s_and_b64 vcc, vcc, {sr(S_M2, 2)}")
            x = s_cur + 16 * qb + a
            b.emit(f"v_cndmask_b32 {vr(x)}, {vr(VNINF)}, {vr(x)}, vcc")
    b.emit(f"{skip_label}:")


def slow_path(b: Block, s_cur, p_cur, c, label, ret):
    """Raise m to the sub-tile maximum, rescale O and l, recompute P and the sums."""
    b.emit(f"{label}:")
    b.emit("s_nop 7")
    b.emit("s_nop 7")
    b.emit("s_nop 7")
    for qb in range(2):
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
        b.emit(f"v_mul_f32 {vr(VL[qb])}, {vr(VL[qb])}, {vr(al)}")
        tmps = [X0 + 4, X0 + 5, X0 + 6, X0 + 7]
        for i in range(64):
            acc = 64 * qb + i
            t = tmps[i % 4]
            b.emit(f"v_accvgpr_read_b32 {vr(t)}, {ar(acc)}")
            b.emit(f"v_mul_f32 {vr(t)}, {vr(t)}, {vr(al)}")
            b.emit(f"v_accvgpr_write_b32 {ar(acc)}, {vr(t)}")
    for ln in softmax_ops(s_cur, p_cur, c):
        b.emit(ln)
    b.emit(f"s_branch {ret}")


def tile_of(b: Block, dst: int, idx_reg: str):
    """dst = idx < a_end ? idx : b_start + idx - a_end."""
    b.emit(f"s_sub_u32 {sr(S_TMP)}, {idx_reg}, %[a_end]")
    b.emit(f"s_add_u32 {sr(S_TMP)}, {sr(S_TMP)}, %[b_start]")
    b.emit(f"s_cmp_lt_u32 {idx_reg}, %[a_end]")
    b.emit(f"s_cselect_b32 {sr(dst)}, {idx_reg}, {sr(S_TMP)}")


def dma(b: Block, kt_reg: int, is_k: bool, lds_byte: int, dpw: int):
    """LDS-direct loads of one 64-key tile (this wave's rows) to LDS byte offset lds_byte."""
    base_lo, base_hi = ("%[kb_lo]", "%[kb_hi]") if is_k else ("%[vb_lo]", "%[vb_hi]")
    b.emit(f"s_mul_i32 {sr(S_OFF)}, {sr(kt_reg)}, %[rb64]")
    b.emit(f"s_add_u32 {sr(S_RSRC)}, {base_lo}, {sr(S_OFF)}")
    b.emit(f"s_addc_u32 {sr(S_RSRC + 1)}, {base_hi}, 0")
    b.emit(f"s_sub_u32 {sr(S_RSRC + 2)}, %[nrec], {sr(S_OFF)}")
    b.emit(f"s_mov_b32 {sr(S_RSRC + 3)}, 0x20000")
    b.emit(f"s_mov_b32 {sr(S_SO)}, %[wsoff]")
    for i in range(dpw):
        b.emit(f"s_add_u32 m0, %[wlds], {lds_byte + 1024 * i}")
        if i:
            b.emit(f"s_add_u32 {sr(S_SO)}, {sr(S_SO)}, %[rb4]")
        else:
            b.emit("s_nop 0")
        voff = f"%[ko{i % 4}]" if is_k else "%[vo]"
        b.emit(f"buffer_load_dwordx4 {voff}, {sr(S_RSRC, 4)}, {sr(S_SO)} offen lds")


def dma_if(b: Block, vis_add: int, is_k: bool, lds_byte: int, dpw: int, lab: str, count: bool):
    """Loads of visit S_T + vis_add (when it exists); adds dpw to S_NL when `count`."""
    b.emit(f"s_add_u32 {sr(S_NV1)}, {sr(S_T)}, {vis_add}")
    b.emit(f"s_cmp_lt_u32 {sr(S_NV1)}, %[nvis]")
    b.emit(f"s_cbranch_scc0 {lab}")
    tile_of(b, S_LAST, sr(S_NV1))
    dma(b, S_LAST, is_k, lds_byte, dpw)
    if count:
        b.emit(f"s_add_u32 {sr(S_NL)}, {sr(S_NL)}, {dpw}")
    b.emit(f"{lab}:")


def wait_loads(b: Block, dpw: int, stages: int, lab: str):
    """Wait for every load but those issued at the previous barrier (S_NL of them)."""
    if stages == 2:
        b.emit("s_waitcnt vmcnt(0)")
        return
    b.emit(f"s_cmp_eq_u32 {sr(S_NL)}, {2 * dpw}")
    b.emit(f"s_cbranch_scc1 {lab}_w2")
    b.emit(f"s_cmp_eq_u32 {sr(S_NL)}, {dpw}")
    b.emit(f"s_cbranch_scc1 {lab}_w1")
    b.emit("s_waitcnt vmcnt(0)")
    b.emit(f"s_branch {lab}_wd")
    b.emit(f"{lab}_w1:")
    b.emit(f"s_waitcnt vmcnt({dpw})")
    b.emit(f"s_branch {lab}_wd")
    b.emit(f"{lab}_w2:")
    b.emit(f"s_waitcnt vmcnt({2 * dpw})")
    b.emit(f"{lab}_wd:")


def barrier_dma(b: Block, tp: int, dpw: int, stages: int, lab: str):
    """At tile t' = S_T + tp: wait for the loads tile t' still needs, barrier
    (every wave is done with K(t') and V(t'-1)), then load K(t' + STAGES) into
    K stage tp and V(t' + STAGES - 1) into V stage tp - 1."""
    wait_loads(b, dpw, stages, lab)
    b.emit("s_barrier")
    b.emit(f"s_mov_b32 {sr(S_NL)}, 0")
    dma_if(b, tp + stages, True, k_off(tp), dpw, f"{lab}_nok", True)
    dma_if(b, tp + stages - 1, False, v_lds((tp - 1) % stages, stages), dpw, f"{lab}_nov", True)


def pv_tail(b: Block, p_prev: int, voff: int):
    b.reset_ds()
    for f in range(8):
        ks, db = divmod(f, 4)
        buf = VB[f % 3]
        off = voff + 4096 * ks
        b.ds_op(f"v{f}", f"ds_read_b64_tr_b16 {vr(buf, 2)}, %[va{db}] offset:{off}")
        b.ds_op(f"v{f}", f"ds_read_b64_tr_b16 {vr(buf + 2, 2)}, %[va{db}] offset:{off + 2048}")
        if f >= 2:
            g = f - 2
            gks, gdb = divmod(g, 4)
            b.wait_ds(f"v{g}")
            for qb in range(2):
                o = ar(16 * (4 * qb + gdb), 16)
                b.emit(f"{MFMA} {o}, {vr(VB[g % 3], 4)}, {vr(p_prev + 8 * qb + 4 * gks, 4)}, {o}")
    for g in (6, 7):
        gks, gdb = divmod(g, 4)
        b.wait_ds(f"v{g}")
        for qb in range(2):
            o = ar(16 * (4 * qb + gdb), 16)
            b.emit(f"{MFMA} {o}, {vr(VB[g % 3], 4)}, {vr(p_prev + 8 * qb + 4 * gks, 4)}, {o}")


def loop_block(dpw: int, stages: int) -> list[str]:
    b = Block()
    c = "%[c]"
    b.emit("s_waitcnt vmcnt(0) lgkmcnt(0)")
    # ---- init
    for i in range(128):
        b.emit(f"v_accvgpr_write_b32 {ar(i)}, 0")
    for i in range(16):
        b.emit(f"v_mov_b32 {vr(P_B + i)}, 0")
    for qb in range(2):
        b.emit(f"v_mov_b32 {vr(VM[qb])}, 0xf149f2ca")  # -1e30
        b.emit(f"v_mov_b32 {vr(VL[qb])}, 0")
    b.emit(f"v_mov_b32 {vr(VNINF)}, 0xff800000")
    b.emit(f"s_mov_b32 {sr(S_LIM)}, 0x4b800000")  # 2^24
    b.emit(f"s_mov_b32 {sr(S_T)}, 0")
    # ---- prologue: K(0 .. STAGES-1) and V(0 .. STAGES-2), the loads the
    # barriers of visits -STAGES+1 .. -1 would have issued; then QK(0) -> S_A
    for v in range(stages):
        dma_if(b, v, True, k_off(v), dpw, f"L_prok{v}", False)
    for v in range(stages - 1):
        dma_if(b, v, False, v_lds(v, stages), dpw, f"L_prov{v}", False)
    b.emit("s_waitcnt vmcnt(0)")
    b.emit(f"s_mov_b32 {sr(S_NL)}, 0")
    b.emit("s_barrier")
    b.reset_ds()
    for ds in range(8):
        b.ds_op(f"k{ds}", f"ds_read_b128 {vr(KB[ds % 3], 4)}, %[ka{ds}] offset:{k_off(0)}")
        if ds >= 2:
            g = ds - 2
            b.wait_ds(f"k{g}")
            for qb in range(2):
                acc = vr(S_A + 16 * qb, 16)
                b.emit(f"{MFMA} {acc}, {vr(KB[g % 3], 4)}, {ar(128 + 32 * qb + 4 * g, 4)}, "
                       f"{'0' if g == 0 else acc}")
    for g in (6, 7):
        b.wait_ds(f"k{g}")
        for qb in range(2):
            acc = vr(S_A + 16 * qb, 16)
            b.emit(f"{MFMA} {acc}, {vr(KB[g % 3], 4)}, {ar(128 + 32 * qb + 4 * g, 4)}, {acc}")
    for _ in range(3):
        b.emit("s_nop 7")
    # ---- main loop over groups of STAGES tiles (S_T a multiple of STAGES at the top)
    b.emit("L_loop:")
    pos = 0
    slow = []
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
            else:  # QK: first half of tile t' + 1; PV: first half of tile t'
                koff = k_off((tp + 1) % stages)
                voff = v_off(tp)
            b.emit(f"s_add_u32 {sr(S_NV1)}, {sr(S_T)}, {tp}")
            b.emit(f"s_cmp_ge_u32 {sr(S_NV1)}, %[a_full]")
            b.emit(f"s_cbranch_scc0 L_nomask{pos}")
            mask_code(b, s_cur, h, f"L_nomask{pos}")
            b.emit("s_waitcnt lgkmcnt(0)")
            step(b, s_cur, s_next, p_cur, p_prev, koff, voff, c)
            b.emit(f"v_cmp_lt_f32 vcc, {sr(S_LIM)}, {vr(VT[0])}")
            b.emit(f"v_cmp_lt_f32 {sr(S_M2, 2)}, {sr(S_LIM)}, {vr(VT[1])}")
            b.emit(f"s_or_b64 vcc, vcc, {sr(S_M2, 2)}")
            b.emit(f"s_cbranch_vccnz L_slow{pos}")
            b.emit(f"L_ret{pos}:")
            b.emit(f"v_add_f32 {vr(VL[0])}, {vr(VL[0])}, {vr(VT[0])}")
            b.emit(f"v_add_f32 {vr(VL[1])}, {vr(VL[1])}, {vr(VT[1])}")
            slow.append((s_cur, p_cur, f"L_slow{pos}", f"L_ret{pos}"))
            if h == 0:
                barrier_dma(b, tp, dpw, stages, f"L_bar{pos}")
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
    for _ in range(3):
        b.emit("s_nop 7")
    b.emit(f"v_mov_b32 %[l0], {vr(VL[0])}")
    b.emit(f"v_mov_b32 %[l1], {vr(VL[1])}")
    b.emit("s_branch L_end")
    for args in slow:
        slow_path(b, *args[:2], c, *args[2:])
    b.emit("L_end:")
    return [ln for ln in b.lines if ln]


def clobbers() -> list[str]:
    regs = [f'"v{i}"' for i in range(NUM_V)]
    regs += [f'"s{i}"' for i in SGPRS]
    regs += ['"vcc"', '"scc"', '"m0"', '"memory"']
    return regs


HEADER = """// Generated by gen_attn_loop.py; do not edit by hand.
// The key-tile loop of the bf16 MIS attention kernel as one gfx950 asm block
// (register map and pipeline: see gen_attn_loop.py).
"""


def render() -> str:
    out = [HEADER]
    for dpw, stages in ((4, 3), (8, 2)):
        lines = loop_block(dpw, stages)
        # labels must be unique per asm instance: %= expands to a per-instance number
        text = []
        for ln in lines:
            ln = ln.replace("L_", "L%=_")
            text.append(f'  "{ln}\\n"')
        out.append(f"#define MIS_ATTN_LOOP_TEXT_DPW{dpw} \\")
        out.append(" \\\n".join(text))
        out.append("")
    out.append("#define MIS_ATTN_LOOP_CLOBBERS " + ", ".join(clobbers()))
    out.append("")
    return "\n".join(out)


def main():
    with open(OUT, "w") as f:
        f.write(render())


if __name__ == "__main__":
    main()
