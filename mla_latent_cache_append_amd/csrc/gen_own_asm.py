"""Writes own_asm.inc: the instruction sequences of the 128-row attention
kernel's inner loop (attn_own_kernel in attn.hip), as inline-asm templates.

The loop body is emitted instruction by instruction so that the schedule is
exactly the one intended: LDS operand reads issued several MFMAs ahead of
their use with exact lgkmcnt waits, the softmax VALU work interleaved with
the MFMAs, and no register traffic between the accumulators and VGPRs.
Values that live across iterations (query fragments, the masked scores of
the next half tile, the running max and sum, the PV accumulators, LDS
addresses) are named operands allocated by the compiler; values that live
only inside one iteration (the score accumulator, the K and V^T fragment
rings, the packed probabilities, temporaries) sit in fixed registers listed
as clobbers.

Templates (iteration e scores half tile e+1 and accumulates half tile e):
  OWN_ASM_QLOAD
        start of a segment: copies of its first three half tiles with the
        query fragments loaded in between, waiting for the first half tile
        and the fragments
  OWN_ASM_PRO
        scores of the first half tile of a segment (36 k-steps), then the
        first half of its softmax (key mask, row max, rescale factor, new
        running max, reference mref); the masked scores go to s0..s15
  OWN_ASM_IT, OWN_ASM_IT_FIRST
        phase S: the 36 score MFMAs of half tile e+1 carrying the second half
                 of the softmax of half tile e (probabilities 2^(s scale -
                 mref), row sum into l after alpha, bf16 packing into P);
        phase P: the 32 PV MFMAs of half tile e,
                 O^T[col][row] += V^T[col][token] P^T[token][row], V^T
                 fragments read transposed, carrying the first half of the
                 softmax of half tile e+1 (with the key mask; IT skips
                 the mask when operand `open` is non-zero: a half tile
                 whose keys every row may see);
        nine buffer -> LDS copies of this wave's share of half tile e+3 are
        spread over phase S; FIRST starts the PV accumulators from zero.
        These end with PV MFMAs still in flight.
  OWN_ASM_GUARD
        wait states after them, before code that reads the accumulators.

The MFMA is v_mfma_f32_32x32x16_bf16 throughout. Run: python gen_own_asm.py
(the build runs it before compiling).
"""

import os

KSTEPS = 36          # 576 features / 16
PF_K = int(os.environ.get("OWN_PF_K", "4"))   # K fragments in flight
PF_V = int(os.environ.get("OWN_PF_V", "5"))   # V^T fragments in flight (two reads each)
NEG_INF = "0xff800000"
HERE = os.path.dirname(os.path.abspath(__file__))

# ---- fixed registers (clobbered by every template), from v255 down
_top = 256
VR0 = _top - 4 * PF_V                      # V^T ring: slot i = v[VR0 + 4i : +3]
VRING = [("v[%d:%d]" % (VR0 + 4 * i, VR0 + 4 * i + 1), "v[%d:%d]" % (VR0 + 4 * i + 2, VR0 + 4 * i + 3),
          "v[%d:%d]" % (VR0 + 4 * i, VR0 + 4 * i + 3)) for i in range(PF_V)]
KR0 = VR0 - 4 * PF_K                       # K ring: slot i = v[KR0 + 4i : +3]
KRING = ["v[%d:%d]" % (KR0 + 4 * i, KR0 + 4 * i + 3) for i in range(PF_K)]
P0 = KR0 - 8                               # packed probabilities, two MFMA operands
P_OP = ["v[%d:%d]" % (P0, P0 + 3), "v[%d:%d]" % (P0 + 4, P0 + 7)]
SN0 = P0 - 16                              # score accumulator of the next half tile
SN = "v[%d:%d]" % (SN0, SN0 + 15)
T0 = SN0 - 4                               # temporaries
TMP = ["v%d" % (T0 + i) for i in range(4)]
CLOB_LO = T0
# MFMA results settle before VALU code reads them (24 wait states: more than an
# 8-pass XDL result needs). Used only where a VALU instruction follows an MFMA
# whose result it reads with no other instructions between; measured, each
# nop wait state costs about four cycles of the wave's issue.
GUARD = ["s_nop 7", "s_nop 7", "s_nop 7"]

# the nine copies of the next stage, one after every fourth score MFMA (the
# vector memory unit takes the four waves' copies one at a time; bunched
# together they stall the issuing waves; issued in phase P they arrive later)
DMA_S = [1, 5, 9, 13, 17, 21, 25, 29, 33]
DMA_P = []
S_VALU_STEPS = int(os.environ.get("OWN_S_VALU", "16"))   # score MFMAs that carry the probability half
EXP_SKEW = int(os.environ.get("OWN_EXP_SKEW", "0"))      # probability i's exp placed after fma i + skew
P_VALU_FROM = 3      # PV MFMA after which the max half of the softmax starts
BOOK_FROM = 4        # PV MFMA after which the scalar bookkeeping starts
PREP_AT = int(os.environ.get("OWN_PREP_AT", "29"))       # PV MFMA before which every LDS read (and the block id) is waited for


class Seq:
    """Instruction list with a model of the in-order LDS counter (lgkmcnt)."""

    def __init__(self):
        self.lines = []
        self.pending = []          # tags of LDS reads not yet waited for, in issue order

    def op(self, s):
        self.lines.append(s)

    def lds(self, s, tag):
        assert len(self.pending) < 15, "too many LDS reads in flight for lgkmcnt"
        self.lines.append(s)
        self.pending.append(tag)

    def need(self, tag):
        if tag not in self.pending:
            return
        i = max(k for k, t in enumerate(self.pending) if t == tag)
        self.lines.append("s_waitcnt lgkmcnt(%d)" % (len(self.pending) - i - 1))
        self.pending = self.pending[i + 1:]

    def drain(self):
        if self.pending:
            self.lines.append("s_waitcnt lgkmcnt(0)")
            self.pending = []

    def text(self):
        return "".join(l + "\\n\\t" for l in self.lines)


def kread(seq, ks):
    """K fragment of k-step ks (token c32, chunk 2 ks + h) into ring slot ks % PF_K."""
    seq.lds("ds_read_b128 %s, %%[ka%d] offset:%d" % (KRING[ks % PF_K], ks & 3, (ks >> 2) * 1024), "K%d" % ks)


def score_mfma(seq, ks):
    seq.need("K%d" % ks)
    seq.op("v_mfma_f32_32x32x16_bf16 %s, %s, %%[q%d], %s" % (SN, KRING[ks % PF_K], ks, "0" if ks == 0 else SN))


def pv_step(j):
    """Column block and token block of PV step j. The 16 column blocks of
    token block 0 come first, then those of token block 1, so an MFMA never
    accumulates onto the result of the one just before it."""
    return j % 16, j // 16


def vread(seq, j):
    """V^T fragment of PV step j: two transposing reads into the two halves
    of ring slot j % PF_V."""
    cb, kk = pv_step(j)
    lo, hi, _ = VRING[j % PF_V]
    seq.lds("ds_read_b64_tr_b16 %s, %%[va%d] offset:%d" % (lo, cb & 1, kk * 18432 + (cb >> 1) * 1024), "V%da" % j)
    seq.lds("ds_read_b64_tr_b16 %s, %%[va%d] offset:%d" % (hi, 2 + (cb & 1), kk * 18432 + 9216 + (cb >> 1) * 1024),
            "V%db" % j)


# Two-buffer cache (PE = True below): the latent rows (1,024 bytes per token)
# and the rope rows (128 bytes per token) sit in two arrays. The 1-KiB copies
# of column groups 0..7 of a half tile read the latent array with the same
# instructions as the pool (operands go / so / rs carry the 1,024-byte
# stride); the copy of column group 8 reads the rope array through its own
# offsets gp / sp and descriptor rp, at instruction offset 0.
PE = False


def pe_line(cg):
    return PE and cg == 8


def dma_m0(seq, cg, mb="mb"):
    """M0 for line cg of this wave's share of a stage. A buffer -> LDS copy
    adds its instruction offset (cg * 128, see dma_load) to the LDS address
    as well as to the memory address, so M0 = line base - cg * 128 and the
    line lands at mb + cg * 1024 (the rope line of the two-buffer cache has
    offset 0). The copy that reads M0 must not be the next instruction (one
    wait state)."""
    seq.op("s_add_u32 m0, %%[%s], 0x%x" % (mb, cg * 1024 if pe_line(cg) else cg * (1024 - 128)))


def dma_load(seq, cg, rs="rs"):
    """Line cg: buffer -> LDS copy of 1 KiB to M0 (the copy counts in vmcnt,
    not lgkmcnt): the wave's 8 tokens (soffset so) at column group cg
    (instruction offset cg * 128). The cache is read once per call, so the
    copy is marked non-temporal (nt): it streams past the caches instead of
    displacing the split partials the merge reads right after (measured ~2 %
    faster per call, same results)."""
    if pe_line(cg):
        seq.op("buffer_load_dwordx4 %%[gp], %%[%s], %%[sp] offen offset:0 nt lds" % rs.replace("rs", "rp"))
    else:
        seq.op("buffer_load_dwordx4 %%[go], %%[%s], %%[so] offen offset:%d nt lds" % (rs, cg * 128))


def dma(seq, cg, mb="mb", rs="rs"):
    """Both halves of a copy, with the wait state between them as a nop."""
    dma_m0(seq, cg, mb)
    seq.op("s_nop 0")
    dma_load(seq, cg, rs)


def sn_reg(i):
    return "v%d" % (SN0 + i)


def softmax_max(mask):
    """First half of the online softmax of one half tile for the lane's row,
    on the score accumulator (value i = token 8 (i / 4) + 4 h + i % 4 of the
    half tile; lr = last visible key minus the token of value 0): key mask,
    row max, the rescale factor alpha of the running state, the new running
    max and the reference mref the probabilities are taken against. The
    masked scores end in s0..s15."""
    t0, t1, t2, ninf = TMP
    v = []
    if mask:
        # v_cndmask reads VCC over the constant bus, so -inf comes from a register
        v.append("v_mov_b32 %s, %s" % (ninf, NEG_INF))
        for i in range(16):   # keys past the row's position -> -inf
            off = 8 * (i >> 2) + (i & 3)
            v.append("v_cmp_le_i32 vcc, %d, %%[lr]" % off)
            v.append("v_cndmask_b32 %%[s%d], %s, %s, vcc" % (i, ninf, sn_reg(i)))
    else:
        for i in range(16):
            v.append("v_mov_b32 %%[s%d], %s" % (i, sn_reg(i)))
    v.append("v_max3_f32 %s, %%[s0], %%[s1], %%[s2]" % t0)
    for i in range(3, 15, 2):
        v.append("v_max3_f32 %s, %s, %%[s%d], %%[s%d]" % (t0, t0, i, i + 1))
    v.append("v_max_f32 %s, %s, %%[s15]" % (t0, t0))
    v.append("v_mov_b32 %s, %s" % (t1, t0))
    v.append("s_nop 1")
    v.append("v_permlane32_swap_b32 %s, %s" % (t0, t1))      # halves of the wave swapped
    v.append("v_max_f32 %s, %s, %s" % (t0, t0, t1))            # row max over both halves
    v.append("v_mul_f32 %s, %s, %%[scale]" % (t0, t0))        # in log2 units
    v.append("v_add_f32 %s, 0x41000000, %%[mrun]" % t1)       # running max + 8
    v.append("v_cmp_gt_f32 vcc, %s, %s" % (t0, t1))
    v.append("v_cndmask_b32 %s, %%[mrun], %s, vcc" % (t2, t0))  # new max
    v.append("v_sub_f32 %s, %%[mrun], %s" % (t1, t2))
    v.append("v_exp_f32 %s, %s" % (t1, t1))
    v.append("v_cmp_neq_f32 vcc, %s, %%[mrun]" % t2)
    v.append("v_cndmask_b32 %%[alpha], 1.0, %s, vcc" % t1)     # 1 unless the max moved
    v.append("v_mov_b32 %%[mrun], %s" % t2)
    v.append("v_cmp_neq_f32 vcc, %s, %s" % (NEG_INF, t2))
    v.append("v_cndmask_b32 %%[mref], 0, %s, vcc" % t2)        # reference: 0 while nothing is visible
    return v


def softmax_exp():
    """Second half: probabilities 2^(s scale - mref), their sum into the
    running l (after alpha), and the bf16 packing into P for the PV MFMAs."""
    tb = TMP[0]
    v = []
    # exp i follows fma i + EXP_SKEW, so that it does not wait on the result
    # of the instruction just before it
    for k in range(16 + EXP_SKEW):
        if k < 16:
            v.append("v_fma_f32 %%[s%d], %%[s%d], %%[scale], -%%[mref]" % (k, k))
        if k >= EXP_SKEW:
            v.append("v_exp_f32 %%[s%d], %%[s%d]" % (k - EXP_SKEW, k - EXP_SKEW))
    v.append("v_add_f32 %s, %%[s0], %%[s1]" % tb)
    for i in range(2, 16):
        v.append("v_add_f32 %s, %s, %%[s%d]" % (tb, tb, i))
    for j in range(8):
        v.append("v_cvt_pk_bf16_f32 v%d, %%[s%d], %%[s%d]" % (P0 + j, 2 * j, 2 * j + 1))
    v.append("v_fma_f32 %%[lrun], %%[lrun], %%[alpha], %s" % tb)
    return v


NEG_STAGES = "0xfffe5000"    # -3 stages of 36,864 bytes: from stage 3 back to stage 0
STAGE = "0x9000"


def book_keeping():
    """Address work for the next sequence, spread over the PV MFMAs (a lone
    wave issues about one instruction per four cycles, so this costs no MFMA
    time here, unlike code between the sequences): the K addresses of the
    next scores (stage e + 2, or e + 1 again past e1), then, after the last
    V^T read, the V^T addresses of the next PV (stage e + 1) and the next
    mask limit. Stage deltas come from the uniform input ep = e + 4 through
    scratch SGPRs; SCC chains are contiguous. Returns (main, tail)."""
    b = [
        "s_sub_i32 %[t0], %[ep], 2",
        "s_and_b32 %[t1], %[t0], 3",
        "s_cmp_eq_u32 %[t1], 0",
        "s_mov_b32 %[t1], " + STAGE,          # (one literal per scalar instruction)
        "s_cselect_b32 %[t1], " + NEG_STAGES + ", %[t1]",
        "s_cmp_lt_i32 %[t0], %[e1]",
        "s_cselect_b32 %[t1], %[t1], 0",
    ] + ["v_add_u32 %%[ka%d], %%[t1], %%[ka%d]" % (q, q) for q in range(4)]
    tail = [
        "v_subrev_u32 %[lr], 32, %[lr]",
        "s_sub_i32 %[t2], %[ep], 3",
        "s_and_b32 %[t2], %[t2], 3",
        "s_cmp_eq_u32 %[t2], 0",
        "s_mov_b32 %[t2], " + STAGE,
        "s_cselect_b32 %[t2], " + NEG_STAGES + ", %[t2]",
    ] + ["v_add_u32 %%[va%d], %%[t2], %%[va%d]" % (q, q) for q in range(4)]
    return b, tail


def blk_load():
    """Block id of half tile ep = e + 4 (the copies the next sequence
    issues): bt[min(ep / 2, ntiles - 1)], a scalar load issued before any
    LDS read of the sequence. While it is outstanding the lgkmcnt waits
    below, counted for the LDS reads alone, wait for one read more than
    needed; the full drain at PV step PREP_AT waits for it."""
    return ["s_lshr_b32 %[t0], %[ep], 1",
            "s_min_i32 %[t0], %[t0], %[nt1]",
            "s_lshl_b32 %[t0], %[t0], 2",
            "s_load_dword %[blk], %[bt], %[t0]"]


def prep_groups():
    """Descriptor (r0..r3) and LDS base (mb) of the copies of half tile
    ep = e + 4 from its block id: base = pool + blk * 73,728 + (ep & 1) *
    36,864 (bits 47..32 in r1), bytes = 1,152 * min(32, L - 32 ep), or 0 past
    the segment (ep >= e1) or for a block id outside the pool, which inside
    the segment sets bd. Groups are emitted whole, so that no other SCC
    writer falls inside a compare / select or carry chain; mb is read by
    the sequence's copies, all issued before these."""
    return [
        ["s_mul_i32 %[r0], %[blk], 0x12000", "s_mul_hi_u32 %[r1], %[blk], 0x12000"],
        ["s_bitcmp1_b32 %[ep], 0", "s_cselect_b32 %[r2], 0x9000, 0"],
        ["s_add_u32 %[r0], %[r0], %[r2]", "s_addc_u32 %[r1], %[r1], 0"],
        ["s_add_u32 %[r0], %[r0], %[plo]", "s_addc_u32 %[r1], %[r1], %[phi]"],
        ["s_and_b32 %[r1], %[r1], 0xffff"],
        ["s_lshl_b32 %[r2], %[ep], 5", "s_sub_i32 %[r2], %[L], %[r2]"],
        ["s_min_i32 %[r2], %[r2], 32", "s_mul_i32 %[r2], %[r2], 0x480"],
        ["s_cmp_ge_u32 %[blk], %[nblk]", "s_cselect_b32 %[r3], 1, 0", "s_cselect_b32 %[r2], 0, %[r2]"],
        ["s_cmp_lt_i32 %[ep], %[e1]", "s_cselect_b32 %[r3], %[r3], 0", "s_cselect_b32 %[r2], %[r2], 0"],
        ["s_or_b32 %[bd], %[bd], %[r3]", "s_mov_b32 %[r3], 0x20000"],
        ["s_and_b32 %[mb], %[ep], 3", "s_mul_i32 %[mb], %[mb], 0x9000", "s_add_u32 %[mb], %[mb], %[mb0]"],
    ]


def prep_groups_pe():
    """Two-buffer cache: descriptors of the copies of half tile ep = e + 4,
    latent rows (r0..r3) at kv + ep * 32,768 and rope rows (r4..r7) at pe +
    ep * 4,096 (the sequence's bases klo:khi and plo:phi, bits 47..32 in the
    second word), bytes = 1,024 (128) * max(0, min(32, Lc - 32 ep)), or 0
    past the segment (ep >= e1); LDS base mb as for the pool. Groups are
    emitted whole (SCC chains)."""
    return [
        ["s_mul_i32 %[r0], %[ep], 0x8000", "s_mul_hi_u32 %[r1], %[ep], 0x8000"],
        ["s_add_u32 %[r0], %[r0], %[klo]", "s_addc_u32 %[r1], %[r1], %[khi]"],
        ["s_and_b32 %[r1], %[r1], 0xffff"],
        ["s_mul_i32 %[r4], %[ep], 0x1000", "s_mul_hi_u32 %[r5], %[ep], 0x1000"],
        ["s_add_u32 %[r4], %[r4], %[plo]", "s_addc_u32 %[r5], %[r5], %[phi]"],
        ["s_and_b32 %[r5], %[r5], 0xffff"],
        ["s_lshl_b32 %[r2], %[ep], 5", "s_sub_i32 %[r2], %[L], %[r2]"],
        ["s_min_i32 %[r2], %[r2], 32", "s_max_i32 %[r2], %[r2], 0"],
        ["s_cmp_lt_i32 %[ep], %[e1]", "s_cselect_b32 %[r2], %[r2], 0"],
        ["s_lshl_b32 %[r6], %[r2], 7", "s_lshl_b32 %[r2], %[r2], 10"],
        ["s_mov_b32 %[r3], 0x20000", "s_mov_b32 %[r7], 0x20000"],
        ["s_and_b32 %[mb], %[ep], 3", "s_mul_i32 %[mb], %[mb], 0x9000", "s_add_u32 %[mb], %[mb], %[mb0]"],
    ]


def gen_qload():
    """Start of a segment: the copies of the first half tile, the 36 query
    fragments straight into registers (row 32 wave + l % 32 at byte offset
    qv, k-step ks at + 32 ks), then the copies of the next two half tiles;
    returns once the first half tile and the fragments have arrived (vector
    memory results count down in issue order)."""
    s = Seq()
    for cg in range(9):
        dma(s, cg, "mb0", "rs0")   # lines of half tile e0
    for ks in range(KSTEPS):
        s.op("buffer_load_dwordx4 %%[q%d], %%[qv], %%[qr], 0 offen offset:%d" % (ks, 32 * ks))
    for st in (1, 2):
        for cg in range(9):
            dma(s, cg, "mb%d" % st, "rs%d" % st)
    s.op("s_waitcnt vmcnt(18)")
    return s.text()


def gen_pro(mask):
    s = Seq()
    s.op("s_nop 1")
    for ks in range(PF_K):
        kread(s, ks)
    for ks in range(KSTEPS):
        score_mfma(s, ks)
        if ks + PF_K < KSTEPS:
            kread(s, ks + PF_K)
    s.lines += GUARD                 # scores settle before the VALU reads them
    s.lines += softmax_max(mask)
    return s.text()


def gen_iter(mask, first):
    """mask: the key mask of the half tile whose scores are formed (needed
    only where some key lies past some row's position). The sequence ends
    with PV MFMAs in flight: code after it that reads the accumulators waits
    first (GUARD)."""
    s = Seq()
    if not PE:
        for ins in blk_load():
            s.op(ins)
    s.op("s_nop 1")
    for ks in range(PF_K):
        kread(s, ks)
    # a few probability instructions cover the latency of the first K read
    exp_valu = softmax_exp()
    lead, rest = exp_valu[:8], exp_valu[8:]
    per = (len(rest) + S_VALU_STEPS - 1) // S_VALU_STEPS
    for ins in lead:
        s.op(ins)
    vnext = 0
    for ks in range(KSTEPS):
        if ks in DMA_S:
            dma_m0(s, DMA_S.index(ks))     # the score MFMA below is the wait state
        score_mfma(s, ks)
        if ks + PF_K < KSTEPS:
            kread(s, ks + PF_K)
        elif vnext < PF_V:                 # K reads done: fill the V^T ring
            vread(s, vnext)
            vnext += 1
        if ks in DMA_S:
            dma_load(s, DMA_S.index(ks))
        for ins in rest[ks * per:(ks + 1) * per]:
            s.op(ins)
    while vnext < PF_V:
        vread(s, vnext)
        vnext += 1
    book, book_tail = book_keeping()
    max_valu = softmax_max(mask)
    nsteps = 32 - P_VALU_FROM - 6
    mper = (len(max_valu) + nsteps - 1) // nsteps
    # bookkeeping from PV step BOOK_FROM on, the V^T address update after the
    # last V^T read (issued at step 31 - PF_V), the rescale test at the end
    bper = (len(book) + (31 - PF_V - BOOK_FROM) - 1) // (31 - PF_V - BOOK_FROM)   # at least one per step
    prep = prep_groups_pe() if PE else prep_groups()
    pper = (len(prep) + (32 - PREP_AT) - 1) // (32 - PREP_AT)
    for j in range(32):
        if j == PREP_AT:
            s.drain()          # the last V^T reads and the block id
        s.need("V%db" % j)
        cb, kk = pv_step(j)
        acc = "0" if first and kk == 0 else "%%[o%d]" % cb   # first half tile: start from 0
        s.op("v_mfma_f32_32x32x16_bf16 %%[o%d], %s, %s, %s" % (cb, VRING[j % PF_V][2], P_OP[kk], acc))
        if j + PF_V < 32:
            vread(s, j + PF_V)
        if j in DMA_P:
            dma(s, len(DMA_S) + DMA_P.index(j))
        # The max half reads the last score MFMA's result only after
        # P_VALU_FROM + 1 PV MFMAs and their V^T reads and waits: more than
        # the 11 wait states an 8-pass result needs before a VALU read, and
        # each of those MFMAs waits for the previous one to leave the XDL
        # pipe (32 cycles), so no nop is needed there.
        if j >= P_VALU_FROM:
            k = j - P_VALU_FROM
            for ins in max_valu[k * mper:(k + 1) * mper]:
                s.op(ins)
        if BOOK_FROM <= j < 31 - PF_V:
            k = j - BOOK_FROM
            for ins in book[k * bper:(k + 1) * bper]:
                s.op(ins)
        if j == 32 - PF_V:
            for ins in book_tail:
                s.op(ins)
        if j >= PREP_AT:       # the next copies' descriptor, under the last PV MFMAs
            for g in prep[(j - PREP_AT) * pper:(j - PREP_AT + 1) * pper]:
                for ins in g:
                    s.op(ins)
    assert (32 - P_VALU_FROM - 6) * mper >= len(max_valu) and (31 - PF_V - BOOK_FROM) * bper >= len(book)
    assert 32 - PF_V < PREP_AT and 31 - PF_V <= PREP_AT and P_VALU_FROM + 32 - P_VALU_FROM - 6 <= PREP_AT
    s.drain()
    return s.text()


# --------------------------------------------------------------- FP8 pool
#
# The FP8 kernel streams E4M3 codes (576 bytes per token) and power-of-two
# token scales into a per-wave staging area and widens them, scale folded in,
# into the same bf16 half-tile stages the products read: code x 2^k is a
# bf16 value, so v_cvt_scalef32_pk_bf16_fp8 gives the row exactly. Stages:
# three bf16 half tiles (slot e % 3: V of e, K of e+1, and e+2 being written)
# and two staging slots per wave (half tiles e+2, being widened, and e+3 in
# flight; e+4 is copied into e+2's slot once it is widened).
#
# Staging slot of a wave: 5,120 bytes of codes (its 8 tokens, 4,608 bytes,
# as five 1 KiB copies; the fifth reads past them) and 256 bytes of scales
# (word i = scale of token min(i, 7)).
F8_STG = 5376
F8_SC_OFF = 5120


def use_layout(pf_k, pf_v, conv):
    """Fixed-register layout (from v255 down) for ring depths pf_k, pf_v and,
    with conv, the FP8 widening registers (two 4-register chunk buffers and
    the lane's token scale)."""
    global PF_K, PF_V, VR0, VRING, KR0, KRING, P0, P_OP, SN0, SN, T0, TMP, CLOB_LO, CB0, CSC
    PF_K, PF_V = pf_k, pf_v
    VR0 = _top - 4 * PF_V
    VRING = [("v[%d:%d]" % (VR0 + 4 * i, VR0 + 4 * i + 1), "v[%d:%d]" % (VR0 + 4 * i + 2, VR0 + 4 * i + 3),
              "v[%d:%d]" % (VR0 + 4 * i, VR0 + 4 * i + 3)) for i in range(PF_V)]
    KR0 = VR0 - 4 * PF_K
    KRING = ["v[%d:%d]" % (KR0 + 4 * i, KR0 + 4 * i + 3) for i in range(PF_K)]
    P0 = KR0 - 8
    P_OP = ["v[%d:%d]" % (P0, P0 + 3), "v[%d:%d]" % (P0 + 4, P0 + 7)]
    SN0 = P0 - 16
    SN = "v[%d:%d]" % (SN0, SN0 + 15)
    T0 = SN0 - 4
    TMP = ["v%d" % (T0 + i) for i in range(4)]
    CLOB_LO = T0
    CB0 = CSC = None
    if conv:
        CB0 = T0 - 10         # chunk buffers v[CB0 .. CB0+7] (even: 64-bit tuples), scale v[CB0+8]
        CSC = "v%d" % (CB0 + 8)
        CLOB_LO = CB0


F8_HT_NEG2 = "0xfffee000"    # -2 stages of 36,864 bytes: from stage 2 back to stage 0


def conv_read(seq, c):
    """Codes of chunk group c of the lane's token (8 bytes at the read base
    + 64 c) into the upper half of chunk buffer c % 2."""
    b = CB0 + 4 * (c % 2)
    seq.lds("ds_read_b64 v[%d:%d], %s offset:%d" % (b + 2, b + 3, TMP[1], 64 * c), "C%d" % c)


def conv_widen(seq, c):
    """Four conversions (two codes each, scale folded in) into the whole
    buffer, in an order that overwrites each code register only after its
    last use, then the 16-byte write into the bf16 stage (cw + 1,024 c)."""
    b = CB0 + 4 * (c % 2)
    seq.need("C%d" % c)
    seq.op("v_cvt_scalef32_pk_bf16_fp8 v%d, v%d, %s" % (b, b + 2, CSC))
    seq.op("v_cvt_scalef32_pk_bf16_fp8 v%d, v%d, %s op_sel:[1,0,0]" % (b + 1, b + 2, CSC))
    seq.op("v_cvt_scalef32_pk_bf16_fp8 v%d, v%d, %s" % (b + 2, b + 3, CSC))
    seq.op("v_cvt_scalef32_pk_bf16_fp8 v%d, v%d, %s op_sel:[1,0,0]" % (b + 3, b + 3, CSC))
    seq.lds("ds_write_b128 %s, v[%d:%d] offset:%d" % (TMP[2], b, b + 3, 1024 * c), "W%d" % c)


def dma8_ops(prologue=False):
    """Copies of half tile e+4 into the staging slot just widened (M0 = mb8):
    five 1 KiB code copies (the lane's 16 bytes at so8 + 1,024 c + go8,
    go8 = 16 l; the fifth through go8 + 4,096, since an instruction offset
    stops at 4,095) and the 64 scales of the half tile's block (lane l reads
    scale l at sb + 4 l). The offsets of the last two sit in the chunk
    buffers, free once the widening is done. Each M0 write has one other
    instruction between it and its copy."""
    if prologue:   # outside the loop the two offsets come in as operands
        return [
            ("m0", "s_mov_b32 m0, %[mb8]"),
            ("ld", "buffer_load_dwordx4 %[go8], %[rs], %[so8] offen offset:0 nt lds"),
            ("ld", "buffer_load_dwordx4 %[go8], %[rs], %[so8] offen offset:1024 nt lds"),
            ("ld", "buffer_load_dwordx4 %[go8], %[rs], %[so8] offen offset:2048 nt lds"),
            ("ld", "buffer_load_dwordx4 %[go8], %[rs], %[so8] offen offset:3072 nt lds"),
            ("m0", "s_add_u32 m0, %%[mb8], 0x%x" % 4096),
            ("ld", "buffer_load_dwordx4 %[go8b], %[rs], %[so8] offen offset:0 nt lds"),
            ("m0", "s_add_u32 m0, %%[mb8], 0x%x" % F8_SC_OFF),
            ("ld", "global_load_lds_dword %[soff], %[sb] offset:0"),
        ]
    gb, so = "v%d" % CB0, "v%d" % (CB0 + 1)
    return [
        ("m0", "s_mov_b32 m0, %[mb8]"),
        ("ld", "buffer_load_dwordx4 %[go8], %[rs], %[so8] offen offset:0 nt lds"),
        ("ld", "buffer_load_dwordx4 %[go8], %[rs], %[so8] offen offset:1024 nt lds"),
        ("ld", "buffer_load_dwordx4 %[go8], %[rs], %[so8] offen offset:2048 nt lds"),
        ("ld", "buffer_load_dwordx4 %[go8], %[rs], %[so8] offen offset:3072 nt lds"),
        ("m0", "s_add_u32 m0, %%[mb8], 0x%x" % 4096),
        ("va", "v_add_u32 %s, 0x1000, %%[go8]" % gb),
        ("ld", "buffer_load_dwordx4 %s, %%[rs], %%[so8] offen offset:0 nt lds" % gb),
        ("m0", "s_add_u32 m0, %%[mb8], 0x%x" % F8_SC_OFF),
        ("va", "v_lshrrev_b32 %s, 2, %%[go8]" % so),
        ("ld", "global_load_lds_dword %s, %%[sb] offset:0" % so),
    ]


def book_keeping8():
    """Address work for the next sequence: K addresses to the stage of e+2
    (or e+1 again past e1), V^T addresses to the stage of e+1, and the mask
    limit. Stages advance one slot (+36,864) or wrap from slot 2 to 0;
    r3 = e % 3 says which address wraps. Returns (groups, tail):
    each group is emitted in one piece, so that no SCC-writing instruction
    (the copies' M0 sums) falls between a compare and its select."""
    groups = [
        ["s_sub_i32 %[t0], %[ep], 2",
         "s_cmp_eq_u32 %[r3], 1",
         "s_mov_b32 %[t1], " + STAGE,
         "s_cselect_b32 %[t1], " + F8_HT_NEG2 + ", %[t1]",
         "s_cmp_lt_i32 %[t0], %[e1]",
         "s_cselect_b32 %[t1], %[t1], 0"],
    ] + [["v_add_u32 %%[ka%d], %%[t1], %%[ka%d]" % (q, q)] for q in range(4)]
    tail = [
        "v_subrev_u32 %[lr], 32, %[lr]",
        "s_cmp_eq_u32 %[r3], 2",
        "s_mov_b32 %[t2], " + STAGE,
        "s_cselect_b32 %[t2], " + F8_HT_NEG2 + ", %[t2]",
    ] + ["v_add_u32 %%[va%d], %%[t2], %%[va%d]" % (q, q) for q in range(4)]
    return groups, tail


CONV_AT = [1 + 3 * c for c in range(9)]     # score step after which chunk c is read
DMA8_P = [8, 10, 12, 14, 16, 18, 20, 22, 24, 26, 27]   # PV steps after which the copies go


def gen_iter8(mask, first):
    """FP8 iteration e: as gen_iter (phase S: scores of e+1 under the
    probabilities of e; phase P: PV of e under the max half of e+1), plus the
    widening of half tile e+2 (this wave's 8 tokens) spread over phase S and
    the copies of e+4 in phase P, after the widening has read its slot."""
    s = Seq()
    s.op("s_nop 1")
    for ks in range(PF_K):
        kread(s, ks)
    # widening bases: codes at mb8 + rdo (the lane's swizzled chunk of its
    # token), bf16 stage at cwb + go8; the lane's token scale is word
    # 32 (e & 1) + tlw of the block's 64 in the staging slot, 1 for a token
    # past the half tile's valid ones (its codes are zeros; a scale slot
    # never written might hold anything)
    s.op("v_add_u32 %s, %%[mb8], %%[rdo]" % TMP[1])
    s.op("v_add_u32 %s, %%[cwb], %%[go8]" % TMP[2])
    s.op("s_bitcmp1_b32 %[ep], 0")
    s.op("s_cselect_b32 %[t0], 0x80, 0")
    s.op("s_add_u32 %[t0], %[t0], %[mb8]")
    s.op("v_lshl_add_u32 %s, %%[tlw], 2, %%[t0]" % CSC)
    s.lds("ds_read_b32 %s, %s offset:%d" % (CSC, CSC, F8_SC_OFF), "SC")
    exp_valu = softmax_exp()
    lead, rest = exp_valu[:8], exp_valu[8:]
    per = (len(rest) + S_VALU_STEPS - 1) // S_VALU_STEPS
    for ins in lead:
        s.op(ins)
    vnext = 0
    widened = 0
    for ks in range(KSTEPS):
        score_mfma(s, ks)
        if ks + PF_K < KSTEPS:
            kread(s, ks + PF_K)
        elif vnext < PF_V:
            vread(s, vnext)
            vnext += 1
        if ks == 2:
            s.need("SC")
            s.op("v_cmp_gt_i32 vcc, %[nv2], %[tlw]")
            s.op("v_cndmask_b32 %s, 1.0, %s, vcc" % (CSC, CSC))
        if ks in CONV_AT:
            c = CONV_AT.index(ks)
            conv_read(s, c)
            if c >= 1:
                conv_widen(s, c - 1)
                widened = c
        for ins in rest[ks * per:(ks + 1) * per]:
            s.op(ins)
    conv_widen(s, 8)
    while vnext < PF_V:
        vread(s, vnext)
        vnext += 1
    book, book_tail = book_keeping8()
    max_valu = softmax_max(mask)
    nsteps = 32 - P_VALU_FROM - 6
    mper = (len(max_valu) + nsteps - 1) // nsteps
    assert len(book) <= 31 - PF_V - BOOK_FROM
    dma = dma8_ops()
    assert len(dma) == len(DMA8_P)
    for j in range(32):
        s.need("V%db" % j)
        cb, kk = pv_step(j)
        acc = "0" if first and kk == 0 else "%%[o%d]" % cb
        s.op("v_mfma_f32_32x32x16_bf16 %%[o%d], %s, %s, %s" % (cb, VRING[j % PF_V][2], P_OP[kk], acc))
        if j + PF_V < 32:
            vread(s, j + PF_V)
        if j in DMA8_P:
            k = DMA8_P.index(j)
            s.op(dma[k][1])
        if j >= P_VALU_FROM:
            k = j - P_VALU_FROM
            for ins in max_valu[k * mper:(k + 1) * mper]:
                s.op(ins)
        if BOOK_FROM <= j < BOOK_FROM + len(book):
            for ins in book[j - BOOK_FROM]:
                s.op(ins)
        if j == 32 - PF_V:
            for ins in book_tail:
                s.op(ins)
    assert (32 - P_VALU_FROM - 6) * mper >= len(max_valu)
    s.drain()
    return s.text()


def gen_qload8():
    """Start of an FP8 segment: copies of half tiles e0 and e0+1 (codes and
    scales) into the wave's two staging slots, with the 36 query fragments
    loaded between them; waits for all of it (the caller then widens both)."""
    s = Seq()
    for st in (0, 1):
        for kind, text in dma8_ops(prologue=True):
            s.op(text.replace("%[mb8]", "%%[mb%d]" % st).replace("%[rs]", "%%[rs%d]" % st)
                 .replace("%[sb]", "%%[sb%d]" % st))
            if kind == "m0":
                s.op("s_nop 0")
        if st == 0:
            for ks in range(KSTEPS):
                s.op("buffer_load_dwordx4 %%[q%d], %%[qv], %%[qr], 0 offen offset:%d" % (ks, 32 * ks))
    s.op("s_waitcnt vmcnt(0)")
    return s.text()


def gen_copy8():
    """Copies of two half tiles (codes and scales) into the two staging slots."""
    s = Seq()
    for st in (0, 1):
        for kind, text in dma8_ops(prologue=True):
            s.op(text.replace("%[mb8]", "%%[mb%d]" % st).replace("%[rs]", "%%[rs%d]" % st)
                 .replace("%[sb]", "%%[sb%d]" % st))
            if kind == "m0":
                s.op("s_nop 0")
    return s.text()


def main():
    out = os.path.join(HERE, "own_asm.inc")
    body = ["// Generated by gen_own_asm.py; do not edit.", ""]
    # IT_NOMASK serves the half tiles every row sees whole (most of them);
    # IT (key mask) the last ones of a sequence and the causal block
    # (one asm statement holding both, chosen by a scalar branch, so that the
    # loop has a single call site and one register assignment)
    it_sel = ("s_sub_i32 %[t0], %[ep], 3\\n\\ts_cmp_lt_i32 %[t0], %[eo]\\n\\t"
              "s_cbranch_scc1 own_open_%=\\n\\t" + gen_iter(True, False)
              + "s_branch own_done_%=\\n\\town_open_%=:\\n\\t" + gen_iter(False, False) + "own_done_%=:\\n\\t")
    temps = [("OWN_ASM_QLOAD", gen_qload()), ("OWN_ASM_PRO", gen_pro(True)), ("OWN_ASM_IT", it_sel),
             ("OWN_ASM_IT_FIRST", gen_iter(True, True)),
             ("OWN_ASM_GUARD", "".join(l + "\\n\\t" for l in GUARD))]
    for name, text in temps:
        body.append('#define %s "%s"' % (name, text))
        body.append("")
    # operand lists (names of attn_own_kernel's variables)
    ops = {
        "OWN_OPS_Q": ", ".join('[q%d] "v"(qf[%d])' % (i, i) for i in range(KSTEPS)),
        "OWN_OPS_Q_OUT": ", ".join('[q%d] "=&v"(qf[%d])' % (i, i) for i in range(KSTEPS)),
        "OWN_OPS_KA": ", ".join('[ka%d] "v"(ka[%d])' % (i, i) for i in range(4)),
        "OWN_OPS_KA_IO": ", ".join('[ka%d] "+v"(ka[%d])' % (i, i) for i in range(4)),
        "OWN_OPS_VA_IO": ", ".join('[va%d] "+v"(va[%d])' % (i, i) for i in range(4)),
        # bookkeeping operands: scratch SGPRs (outputs never read), then uniform inputs
        "OWN_OPS_BOOK_OUT": '[t0] "=&s"(t0), [t1] "=&s"(t1), [t2] "=&s"(t2)',
        "OWN_OPS_BOOK_IN": '[ep] "s"(e + OSTAGE), [eo] "s"(e_open), [e1] "s"(e1)',
        # the next copies' descriptor: outputs (r0..r3 form rs; blk is scratch) and inputs
        "OWN_OPS_PREP_OUT": ('[r0] "=&s"(r0), [r1] "=&s"(r1), [r2] "=&s"(r2), [r3] "=&s"(r3), '
                             '[blk] "=&s"(blkv), [bd] "+s"(badacc), [mb] "+s"(mb)'),
        "OWN_OPS_PREP_IN": ('[bt] "s"(bt_u), [nt1] "s"(nt1), [plo] "s"(pool_lo), [phi] "s"(pool_hi), '
                            '[L] "s"(L), [nblk] "s"(nblk), [mb0] "s"(mb0)'),
        "OWN_OPS_S_OUT": ", ".join('[s%d] "=&v"(s[%d])' % (i, i) for i in range(16)),
        "OWN_OPS_S": ", ".join('[s%d] "+v"(s[%d])' % (i, i) for i in range(16)),
        "OWN_OPS_O": ", ".join('[o%d] "+a"(o[%d])' % (i, i) for i in range(16)),
        "OWN_OPS_O_OUT": ", ".join('[o%d] "=&a"(o[%d])' % (i, i) for i in range(16)),
        "OWN_OPS_SO": '[so] "s"(so)',
        "OWN_CLOB": ", ".join('"v%d"' % r for r in range(CLOB_LO, 256)),
    }
    for name, text in ops.items():
        body.append("#define %s %s" % (name, text))
    body.append("")
    # two-buffer cache: the same sequences with the rope line read from its
    # own array and the descriptors formed from the half-tile index
    global PE
    PE = True
    it_pe = ("s_sub_i32 %[t0], %[ep], 3\\n\\ts_cmp_lt_i32 %[t0], %[eo]\\n\\t"
             "s_cbranch_scc1 ownp_open_%=\\n\\t" + gen_iter(True, False)
             + "s_branch ownp_done_%=\\n\\townp_open_%=:\\n\\t" + gen_iter(False, False) + "ownp_done_%=:\\n\\t")
    for name, text in [("OWNP_ASM_QLOAD", gen_qload()), ("OWNP_ASM_IT", it_pe),
                       ("OWNP_ASM_IT_FIRST", gen_iter(True, True))]:
        body.append('#define %s "%s"' % (name, text))
        body.append("")
    PE = False
    ops_pe = {
        "OWNP_OPS_PREP_OUT": ('[r0] "=&s"(r0), [r1] "=&s"(r1), [r2] "=&s"(r2), [r3] "=&s"(r3), '
                              '[r4] "=&s"(r4), [r5] "=&s"(r5), [r6] "=&s"(r6), [r7] "=&s"(r7), [mb] "+s"(mb)'),
        "OWNP_OPS_PREP_IN": ('[klo] "s"(kv_lo), [khi] "s"(kv_hi), [plo] "s"(pe_lo), [phi] "s"(pe_hi), '
                             '[L] "s"(Lc), [mb0] "s"(mb0)'),
        "OWNP_OPS_SP": '[gp] "v"(gpoff), [sp] "s"(sp)',
    }
    for name, text in ops_pe.items():
        body.append("#define %s %s" % (name, text))
    body.append("")
    # FP8 pool: the same sequences with shallower operand rings (their
    # registers go to the widening) plus the widening and the code copies
    bf16_layout = (PF_K, PF_V)
    use_layout(3, 3, True)
    it8 = ("s_sub_i32 %[t0], %[ep], 3\\n\\ts_cmp_lt_i32 %[t0], %[eo]\\n\\t"
           "s_cbranch_scc1 own8_open_%=\\n\\t" + gen_iter8(True, False)
           + "s_branch own8_done_%=\\n\\town8_open_%=:\\n\\t" + gen_iter8(False, False) + "own8_done_%=:\\n\\t")
    temps8 = [("OWN8_ASM_QLOAD", gen_qload8()), ("OWN8_ASM_COPY", gen_copy8()), ("OWN8_ASM_PRO", gen_pro(True)),
              ("OWN8_ASM_IT", it8), ("OWN8_ASM_IT_FIRST", gen_iter8(True, True))]
    for name, text in temps8:
        body.append('#define %s "%s"' % (name, text))
        body.append("")
    body.append("#define OWN8_CLOB %s" % ", ".join('"v%d"' % r for r in range(CLOB_LO, 256)))
    body.append("")
    use_layout(*bf16_layout, False)
    new = "\n".join(body)
    if not os.path.exists(out) or open(out).read() != new:
        with open(out, "w") as f:
            f.write(new)
    return out


if __name__ == "__main__":
    print(main())
