"""CPU model of the int8 MFMA fragments the decode and prefill kernels build
(the lane map behind the rule of "Implementing INT8 PV MMAC on a gfx936 DCU",
section 4: one W scale covers exactly the keys one matrix instruction, or one
chain of them, consumes).

The 16x16 int8 MFMAs of CDNA4 (v_mfma_i32_16x16x32_i8: 8 bytes of K per lane;
v_mfma_i32_16x16x64_i8: 16 bytes) take operand A as 16 rows x K and operand B
as K x 16 columns, lane l holding row (resp. column) l % 16 and K-slot block
l / 16, and return D[16][16] with lane l holding column l % 16, rows
4 (l / 16) + i in its four result registers i.  Which K index a (lane block,
byte) slot stands for is the instruction's internal business: since operand
A and operand B of a lane are built from the same key (or head-dim byte) for
the same slot, the dot product over K does not depend on it.  The model below
therefore runs every check under several slot -> K maps (contiguous, split
halves, a random bijection) and requires the same answer under all of them.

Checked, with operands built exactly as the kernels index them:
* prefill QK (S^T = K Q^T, two chains per 32-key group whose A rows read key
  8 (r / 4) + 4 b + r % 4): result register i of lane l in chain b is the score
  of key 8 (l / 16) + 4 b + i of query row l % 16, so a lane holds 8
  consecutive keys of its row;
* prefill PV (O^T = V^T Wq^T): every lane feeds operand B the Wq of exactly
  those 8 keys and operand A the V bytes of the same keys, so one
  16x16x32 MFMA consumes one aligned 32-key group (G = 32) and one 16x16x64
  MFMA one aligned 64-key group (G = 64), and its result is that group's
  sum Wq . Vq;
* decode QK and PV: the page loads put token l % 16 of page 4 g + l / 16 in
  lane l for both Wq (operand A) and V (operand B); with operand A masked to
  lane groups {0, 1} resp. {2, 3} each MFMA consumes one aligned 32-token
  group.
"""
import numpy as np
import pytest

rng = np.random.default_rng(2024)


def slot_maps(kbytes):
    """Candidate (lane block, byte) -> K maps for K = 4 * kbytes."""
    K = 4 * kbytes
    contiguous = {(blk, b): kbytes * blk + b for blk in range(4) for b in range(kbytes)}
    half = kbytes // 2
    split = {(blk, b): (b // half) * (K // 2) + half * blk + b % half
             for blk in range(4) for b in range(kbytes)}
    perm = rng.permutation(K)
    scrambled = {(blk, b): int(perm[kbytes * blk + b]) for blk in range(4) for b in range(kbytes)}
    return {"contiguous": contiguous, "split_halves": split, "bijection": scrambled}


def mfma(A_regs, B_regs, kmap):
    """A 16x16xK int8 MFMA on per-lane byte registers: A_regs[l][b] is
    A[l % 16][kmap[l / 16, b]], B_regs[l][b] is B[kmap[l / 16, b]][l % 16].
    Returns the result registers D_regs[l][i] = D[4 (l / 16) + i][l % 16]."""
    kbytes = A_regs.shape[1]
    K = 4 * kbytes
    A = np.zeros((16, K), np.int64)
    B = np.zeros((K, 16), np.int64)
    seen = set()
    for l in range(64):
        for b in range(kbytes):
            k = kmap[(l // 16, b)]
            seen.add((l % 16, k))
            A[l % 16, k] = A_regs[l, b]
            B[k, l % 16] = B_regs[l, b]
    assert len(seen) == 16 * K, "slot map is not a bijection"
    D = A @ B
    return np.array([[D[4 * (l // 16) + i, l % 16] for i in range(4)] for l in range(64)])


@pytest.mark.parametrize("layout", ["contiguous", "split_halves", "bijection"])
def test_prefill_qk_lane_holds_eight_consecutive_keys(layout):
    D = 256
    kmap = slot_maps(16)[layout]
    keys = rng.integers(-127, 128, (64, D))      # one 64-key tile
    queries = rng.integers(-127, 128, (16, D))   # the wave's 16 rows
    for g in range(2):
        got = np.zeros((64, 8), np.int64)        # lane -> its 8 scores
        for b in range(2):
            acc = np.zeros((64, 4), np.int64)
            for c in range(D // 64):
                A = np.zeros((64, 16), np.int64)
                B = np.zeros((64, 16), np.int64)
                for l in range(64):
                    lr, lg = l % 16, l // 16
                    krow = 32 * g + 8 * (lr >> 2) + 4 * b + (lr & 3)   # key of A row lr
                    A[l] = keys[krow, 64 * c + 16 * lg: 64 * c + 16 * lg + 16]
                    B[l] = queries[lr, 64 * c + 16 * lg: 64 * c + 16 * lg + 16]
                acc += mfma(A, B, kmap)
            got[:, 4 * b: 4 * b + 4] = acc
        for l in range(64):
            lr, lg = l % 16, l // 16
            want = keys[32 * g + 8 * lg: 32 * g + 8 * lg + 8] @ queries[lr]
            assert np.array_equal(got[l], want), (g, l)


@pytest.mark.parametrize("layout", ["contiguous", "split_halves", "bijection"])
@pytest.mark.parametrize("G", [32, 64])
def test_prefill_pv_mfma_consumes_one_aligned_group(layout, G):
    D = 256
    V = rng.integers(-127, 128, (64, D))         # tile keys x dims
    Wq = rng.integers(0, 128, (64, 16))          # tile keys x the wave's 16 rows
    for n in range(D // 16):                     # 16-dim output tile
        dims = slice(16 * n, 16 * n + 16)
        if G == 32:
            kmap = slot_maps(8)[layout]
            for g in range(2):
                A = np.zeros((64, 8), np.int64)
                B = np.zeros((64, 8), np.int64)
                for l in range(64):
                    lr, lg = l % 16, l // 16
                    # the kernel: V bytes of page 2g + lg/2, dim 16n + lr, tokens
                    # 8 (lg & 1) .. +7 = keys 32g + 8lg + j; Wq of its own keys
                    page, off = 2 * g + (lg >> 1), 8 * (lg & 1)
                    A[l] = V[16 * page + off: 16 * page + off + 8, 16 * n + lr]
                    B[l] = Wq[32 * g + 8 * lg: 32 * g + 8 * lg + 8, lr]
                consumed = {32 * g + 8 * (l // 16) + j for l in range(64) for j in range(8)}
                assert consumed == set(range(32 * g, 32 * g + 32))
                got = mfma(A, B, kmap)
                want = V[32 * g: 32 * g + 32, dims].T @ Wq[32 * g: 32 * g + 32]   # [dim, row]
                for l in range(64):
                    for i in range(4):
                        assert got[l, i] == want[4 * (l // 16) + i, l % 16]
        else:
            kmap = slot_maps(16)[layout]
            A = np.zeros((64, 16), np.int64)
            B = np.zeros((64, 16), np.int64)
            for l in range(64):
                lr, lg = l % 16, l // 16
                for h in range(2):   # bytes 8h..8h+7: the lane's 8 keys of 32-key half h
                    page, off = 2 * h + (lg >> 1), 8 * (lg & 1)
                    A[l, 8 * h: 8 * h + 8] = V[16 * page + off: 16 * page + off + 8, 16 * n + lr]
                    B[l, 8 * h: 8 * h + 8] = Wq[32 * h + 8 * lg: 32 * h + 8 * lg + 8, lr]
            consumed = {32 * h + 8 * (l // 16) + j for l in range(64) for h in range(2)
                        for j in range(8)}
            assert consumed == set(range(64))
            got = mfma(A, B, kmap)
            want = V[:, dims].T @ Wq
            for l in range(64):
                for i in range(4):
                    assert got[l, i] == want[4 * (l // 16) + i, l % 16]


@pytest.mark.parametrize("layout", ["contiguous", "split_halves", "bijection"])
@pytest.mark.parametrize("G", [32, 64])
def test_decode_pv_masked_lane_groups_consume_one_group(layout, G):
    """Decode PV over 64 tokens (pages 4g .. 4g+3): operand A = Wq rows (heads)
    with lane group j holding the 16 tokens of page 4g + j, operand B = the V
    row of one dim for the same page; for G = 32 two MFMAs, A masked to lane
    groups {0, 1} and {2, 3}."""
    kmap = slot_maps(16)[layout]
    Wq = rng.integers(0, 128, (16, 64))          # heads x tokens of the 64-token step
    V = rng.integers(-127, 128, (64, 16))        # tokens x 16 dims
    A = np.zeros((64, 16), np.int64)
    B = np.zeros((64, 16), np.int64)
    for l in range(64):
        lr, lg = l % 16, l // 16
        A[l] = Wq[lr, 16 * lg: 16 * lg + 16]
        B[l] = V[16 * lg: 16 * lg + 16, lr]
    groups = [range(0, 64)] if G == 64 else [range(0, 32), range(32, 64)]
    for gi, toks in enumerate(groups):
        Am = A.copy()
        if G == 32:
            keep = (lambda lg: lg < 2) if gi == 0 else (lambda lg: lg >= 2)
            for l in range(64):
                if not keep(l // 16):
                    Am[l] = 0
        got = mfma(Am, B, kmap)
        t = np.array(list(toks))
        want = Wq[:, t] @ V[t]                   # [head, dim]
        for l in range(64):
            for i in range(4):
                assert got[l, i] == want[4 * (l // 16) + i, l % 16]


@pytest.mark.parametrize("layout", ["contiguous", "split_halves", "bijection"])
def test_decode_qk_scores_land_on_head_rows(layout):
    """Decode QK: operand A = the group's queries (row = head, zero-padded to
    16), operand B = one page (lane l: token l % 16, head-dim bytes of chunk
    4c + l / 16); result register r of lane l is head 4 (l / 16) + r, token
    l % 16 -- the index the kernel stores the score under."""
    D = 256
    kmap = slot_maps(16)[layout]
    q = np.zeros((16, D), np.int64)
    q[:6] = rng.integers(-127, 128, (6, D))
    page = rng.integers(-127, 128, (16, D))      # 16 tokens x D
    acc = np.zeros((64, 4), np.int64)
    for c in range(D // 64):
        A = np.zeros((64, 16), np.int64)
        B = np.zeros((64, 16), np.int64)
        for l in range(64):
            lr, lg = l % 16, l // 16
            A[l] = q[lr, 64 * c + 16 * lg: 64 * c + 16 * lg + 16]
            B[l] = page[lr, 64 * c + 16 * lg: 64 * c + 16 * lg + 16]
        acc += mfma(A, B, kmap)
    want = q @ page.T                            # [head, token]
    for l in range(64):
        for r in range(4):
            assert acc[l, r] == want[4 * (l // 16) + r, l % 16]
