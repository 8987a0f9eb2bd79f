"""GPU parity of the demotion (rotate -> clip -> quantize -> pack) against the
oracle: bit-exact packed bytes and bf16 scale/zero given identical rotated
values, and the append/demote state machine of a decode step."""
import numpy as np
import pytest
import torch

import bit_rotated_kv_split_amd as ok
from bit_rotated_kv_split_amd.kvcache import PagedKVCache, Rotation
from oracle import oscar as O
from synth import gen

pytestmark = pytest.mark.gpu


def bits_tensor(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def tensor_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def random_tokens(rng, n, hkv, outlier=True):
    x = rng.standard_normal((n, hkv, 128)).astype(np.float32)
    if outlier:
        x[:, :, [5, 77]] *= 20
    return gen.bf16_bits(x)


def signed_permutation(rng):
    p = O.bit_reversal_matrix(128)
    return (p * rng.choice([-1.0, 1.0], size=128)[None, :]).astype(np.float32)


def make_rot(kind, hkv, rng):
    if kind == "identity":
        rk = np.stack([np.eye(128, dtype=np.float32)] * hkv)
        rv = rk.copy()
    else:
        rk = np.stack([signed_permutation(rng) for _ in range(hkv)])
        rv = np.stack([signed_permutation(rng) for _ in range(hkv)])
    ck = (1.5 + rng.random((hkv, 128))).astype(np.float32) * 2
    cv = (1.0 + rng.random((hkv, 128))).astype(np.float32) * 2
    return rk, rv, ck, cv


CODEBOOK_ID = {"uniform": ok.CODEBOOK_UNIFORM, "lloyd-max": ok.CODEBOOK_LLOYD_MAX}


def slot_bits(slots, group):
    """Mask of the code bits of the given slots in a block (codes 3 and 0
    differ in exactly those bits)."""
    ng = 128 // group
    mine = np.zeros((64, 128), np.uint8)
    mine[slots] = 3
    z = np.zeros((64, ng), np.float32)
    return O.pack_block(mine, z, z, mine, z, z, group) ^ O.pack_block(mine * 0, z, z, mine * 0, z, z, group)


def expected_block(k_bits, v_bits, rk, rv, ck, cv, group, n_valid, codebook="uniform"):
    """Oracle bytes of one page block, zero-filled before, whose first
    n_valid slots hold tokens (the other slots' bits stay 0)."""
    ng = 128 // group
    codes_k = np.zeros((64, 128), dtype=np.uint8)
    codes_v = np.zeros((64, 128), dtype=np.uint8)
    sk = np.zeros((64, ng), np.float32)
    zk = np.zeros((64, ng), np.float32)
    sv = np.zeros((64, ng), np.float32)
    zv = np.zeros((64, ng), np.float32)
    if n_valid:
        c, s, z = O.demote(k_bits[:n_valid], rk, ck, group, codebook)
        codes_k[:n_valid], sk[:n_valid], zk[:n_valid] = c, s, z
        c, s, z = O.demote(v_bits[:n_valid], rv, cv, group, codebook)
        codes_v[:n_valid], sv[:n_valid], zv[:n_valid] = c, s, z
    blk = O.pack_block(codes_k, sk, zk, codes_v, sv, zv, group)
    blk[:4096] &= slot_bits(slice(0, n_valid), group)[:4096]
    return blk


@pytest.mark.parametrize("codebook", ["uniform", "lloyd-max"])
@pytest.mark.parametrize("group", [32, 64, 128])
@pytest.mark.parametrize("kind", ["identity", "signed_perm"])
def test_fill_bit_exact(group, kind, codebook):
    rng = np.random.default_rng(group + (7 if kind == "identity" else 9))
    B, hkv, hq = 2, 2, 4
    n_hist = [150, 64]
    max_pages = 3
    cache = PagedKVCache(hq, hkv, group, B, max_pages, 8, codebook=CODEBOOK_ID[codebook])
    pt = np.array([[5, 0, 3], [7, 2, 6]], dtype=np.int32)
    cache.page_table.copy_(torch.from_numpy(pt))
    cache.seq_lens.copy_(torch.tensor([320 + n for n in n_hist], dtype=torch.int32))
    rk, rv, ck, cv = make_rot(kind, hkv, rng)
    rot = Rotation(rk, rv, ck, cv)
    toks = [(random_tokens(rng, n, hkv), random_tokens(rng, n, hkv)) for n in n_hist]
    for b in range(B):
        kb, vb = toks[b]
        cuts = [0, 37, 100, n_hist[b]] if n_hist[b] > 100 else [0, n_hist[b]]
        for a, e in zip(cuts[:-1], cuts[1:]):
            ok.oscar_kv_fill_history(cache.dims, rot.struct, cache.struct(), b, a, e - a,
                                     bits_tensor(kb[a:e]), bits_tensor(vb[a:e]))
    torch.cuda.synchronize()
    pages = cache.pages.cpu().numpy()
    for b in range(B):
        kb, vb = toks[b]
        for p in range(max_pages):
            n_valid = max(0, min(64, n_hist[b] - 64 * p))
            if n_valid == 0:
                continue
            for j in range(hkv):
                exp = expected_block(kb[64 * p:64 * p + n_valid, j], vb[64 * p:64 * p + n_valid, j],
                                     rk[j], rv[j], ck[j], cv[j], group, n_valid, codebook)
                got = pages[pt[b, p], j]
                assert np.array_equal(got, exp), f"b={b} page={p} kvh={j}"
    # pages no request uses stay zero
    used = set(pt[0, :3].tolist()) | set(pt[1, :1].tolist())
    for q in range(8):
        if q not in used:
            assert not pages[q].any()


@pytest.mark.parametrize("group", [64, 128])
def test_fill_calibrated_rotation_codes(group):
    """With a calibrated (dense) rotation both sides form y = x . R from
    exact products (bf16 x float32 is exact in float64), sum them in float64
    and round once to float32, but in different orders (the GPU's own
    reduction; numpy's BLAS).  The two float64 sums differ by at most about
    2^-46 relative (128 terms, some cancellation), so a rotated value can
    differ in its float32 rounding only when the sum lies within about 2^-22
    float32 ulp of a rounding midpoint: a few values in 10^7, or a few
    percent chance of one among the 262,144 values here.  A scale or zero
    moves only if such a value is its group's minimum or maximum (2 in G)
    and a one-ulp change flips its bf16 rounding (about 2^-16).  So scale/zero must be
    bit-exact here (no group may differ), and codes may differ only within
    1e-5 (relative) of a level boundary, the tolerance the acceptance bar
    states."""
    from synth import configs
    from bit_rotated_kv_split_amd.workload import SyntheticModel
    w = configs.qwen3_8b_b32(group)
    model = SyntheticModel(w)
    q, k, v = model.calibration()
    cal = O.calibrate(q[:, :8], k[:, :2], v[:, :2], w.clip_pct)
    hkv, n = 2, 512
    rng = np.random.default_rng(3)
    cache = PagedKVCache(8, hkv, group, 1, 8, 8)
    cache.page_table.copy_(torch.arange(8, dtype=torch.int32)[None])
    rot = Rotation(cal["r_k32"], cal["r_v32"], cal["clip_k"], cal["clip_v"])
    kb = np.stack([gen.kv_tokens_bf16(w.seed, "k", 0, j, 64, n, model.k_scale[j]) for j in range(hkv)], 1)
    vb = np.stack([gen.kv_tokens_bf16(w.seed, "v", 0, j, 64, n, model.v_scale[j]) for j in range(hkv)], 1)
    del rng
    ok.oscar_kv_fill_history(cache.dims, rot.struct, cache.struct(), 0, 0, n, bits_tensor(kb), bits_tensor(vb))
    torch.cuda.synchronize()
    pages = cache.pages.cpu().numpy()
    sz_mismatch = code_mismatch = 0
    total_groups = 0
    for j in range(hkv):
        for which, bits, r, c in (("k", kb, cal["r_k32"][j], cal["clip_k"][j]),
                                  ("v", vb, cal["r_v32"][j], cal["clip_v"][j])):
            y = O.clip(O.rotate(O.bf16_value(bits[:, j]), r), c)
            codes, s, z = O.quantize_groups(y, group)
            for p in range(n // 64):
                ck_, sk_, zk_, cv_, sv_, zv_ = O.unpack_block(pages[p, j], group)
                gc, gs, gz = (ck_, sk_, zk_) if which == "k" else (cv_, sv_, zv_)
                sl = slice(64 * p, 64 * p + 64)
                bad_g = (gs != s[sl]) | (gz != z[sl])
                sz_mismatch += int(bad_g.sum())
                total_groups += bad_g.size
                # scale/zero within one bf16 step when they differ
                assert np.all(np.abs(gs - s[sl]) <= np.abs(s[sl]) * 2 ** -7)
                assert np.all(np.abs(gz - z[sl]) <= np.abs(z[sl]) * 2 ** -7 + 1e-30)
                ng = 128 // group
                same_g = np.repeat(~bad_g, group, axis=1).reshape(64, 128)
                diff = (gc != codes[sl]) & same_g
                t = (y[sl].astype(np.float64) - np.repeat(z[sl], group, axis=1)) / np.repeat(s[sl], group, axis=1)
                near = np.abs(t - np.floor(t) - 0.5) <= 1e-5 * np.maximum(np.abs(t), 1)
                assert not (diff & ~near).any(), f"kvh={j} {which} page={p}"
                code_mismatch += int(diff.sum())
    assert sz_mismatch == 0, (sz_mismatch, total_groups)


def ring_expect(L, k_all):
    """Expected recent ring [256][128] bits for a request holding L tokens."""
    ring = np.zeros((256, 128), dtype=np.uint16)
    n_r = min(max(L - 64, 0), 256)
    for p in range(L - n_r, L):
        ring[(p - 64) % 256] = k_all[p]
    return ring


@pytest.mark.parametrize("group,codebook", [(32, "uniform"), (128, "uniform"), (64, "lloyd-max")])
def test_decode_steps_append_and_demote(group, codebook):
    """A sequence of decode steps (append + demote) from L = 60 to L = 480
    crosses every region boundary and two page boundaries; the GPU state after
    the last step equals the oracle's: sink and ring bits, packed pages."""
    rng = np.random.default_rng(11 + group)
    B, hkv, hq = 2, 2, 4
    L0, L1 = 60, 480
    start = [L0, L0 + 37]
    total = max(start) + (L1 - L0)
    k_all = random_tokens(rng, total, hkv).reshape(total, hkv, 128)
    k_all = np.stack([k_all, random_tokens(rng, total, hkv)], axis=0)   # [K/V][pos][kvh][128]
    v_all = k_all[1]
    k_all = k_all[0]
    rk, rv, ck, cv = make_rot("signed_perm", hkv, rng)
    rot = Rotation(rk, rv, ck, cv)
    max_pages = 4
    cache = PagedKVCache(hq, hkv, group, B, max_pages, 8, codebook=CODEBOOK_ID[codebook])
    pt = np.array([[4, 1, 2, 6], [0, 5, 3, 7]], dtype=np.int32)
    cache.page_table.copy_(torch.from_numpy(pt))
    # initial state: positions < start[b] as the state machine leaves them
    for b in range(B):
        L = start[b]
        sink = np.zeros((hkv, 64, 128), np.uint16)
        n_s = min(L, 64)
        sink[:, :n_s] = k_all[:n_s].transpose(1, 0, 2)
        cache.sink_k[b] = bits_tensor(sink)
        sink[:, :n_s] = v_all[:n_s].transpose(1, 0, 2)
        cache.sink_v[b] = bits_tensor(sink)
        cache.recent_k[b] = bits_tensor(np.stack([ring_expect(L, k_all[:, j]) for j in range(hkv)]))
        cache.recent_v[b] = bits_tensor(np.stack([ring_expect(L, v_all[:, j]) for j in range(hkv)]))
    lens = np.array(start)
    for step in range(L1 - L0):
        lens = lens + 1
        cache.seq_lens.copy_(torch.from_numpy(lens.astype(np.int32)))
        kn = np.stack([k_all[lens[b] - 1] for b in range(B)])
        vn = np.stack([v_all[lens[b] - 1] for b in range(B)])
        ok.oscar_kv_demote(cache.dims, rot.struct, cache.struct(), bits_tensor(kn), bits_tensor(vn))
    torch.cuda.synchronize()
    pages = cache.pages.cpu().numpy()
    for b in range(B):
        L = int(lens[b])
        assert np.array_equal(tensor_bits(cache.recent_k[b]),
                              np.stack([ring_expect(L, k_all[:, j]) for j in range(hkv)]))
        assert np.array_equal(tensor_bits(cache.recent_v[b]),
                              np.stack([ring_expect(L, v_all[:, j]) for j in range(hkv)]))
        assert np.array_equal(tensor_bits(cache.sink_k[b]), k_all[:64].transpose(1, 0, 2))
        n_hist = L - 320
        for p in range((n_hist + 63) // 64):
            n_valid = min(64, n_hist - 64 * p)
            for j in range(hkv):
                sl = slice(64 + 64 * p, 64 + 64 * p + n_valid)
                exp = expected_block(k_all[sl, j], v_all[sl, j], rk[j], rv[j], ck[j], cv[j], group, n_valid,
                                     codebook)
                assert np.array_equal(pages[pt[b, p], j], exp), f"b={b} page={p} kvh={j}"


def test_demote_only_leaves_ring_alone():
    rng = np.random.default_rng(5)
    hkv = 1
    cache = PagedKVCache(1, hkv, 64, 1, 2, 2)
    cache.page_table.copy_(torch.tensor([[1, 0]], dtype=torch.int32))
    ring = random_tokens(rng, 256, hkv).reshape(256, 128)
    cache.recent_k[0, 0] = bits_tensor(ring)
    cache.recent_v[0, 0] = bits_tensor(ring)
    cache.seq_lens.fill_(321)
    rk, rv, ck, cv = make_rot("identity", hkv, rng)
    rot = Rotation(rk, rv, ck, cv)
    ok.oscar_kv_demote(cache.dims, rot.struct, cache.struct(), None, None)
    torch.cuda.synchronize()
    assert np.array_equal(tensor_bits(cache.recent_k[0, 0]), ring)
    slot = (320 - 256 - 64) % 256   # position 64 -> slot 0
    exp = expected_block(ring[slot:slot + 1], ring[slot:slot + 1], rk[0], rv[0], ck[0], cv[0], 64, 1)
    assert np.array_equal(cache.pages[1, 0].cpu().numpy(), exp)


@pytest.mark.parametrize("codebook", ["uniform", "lloyd-max"])
@pytest.mark.parametrize("group", [32, 64, 128])
def test_fill_degenerate_tokens_bit_exact(group, codebook):
    """Degenerate tokens: all zero, constant within every group (scale 0),
    two-valued groups, values far beyond the clip thresholds (clipped to
    +-c), tiny magnitudes and half-zero tokens.  R = I keeps the rotated
    values exact, so the page bytes must equal the oracle's."""
    rng = np.random.default_rng(50 + group)
    hkv, n = 1, 64
    x = rng.standard_normal((n, hkv, 128)).astype(np.float32)
    x[0] = 0.0
    x[1] *= 1e-3
    x[2] = 1.5
    for gi in range(128 // group):
        x[3, :, gi * group:(gi + 1) * group] = gi - 1.25        # constant per group
    x[4, :, ::2] = 3.0
    x[4, :, 1::2] = -3.0                                          # two-valued groups
    x[5] *= 1e4                                                    # every channel clipped
    x[6, :, :64] = 0.0                                             # half zero
    bits = gen.bf16_bits(x)
    rk, rv, ck, cv = make_rot("identity", hkv, rng)
    rot = Rotation(rk, rv, ck, cv)
    cache = PagedKVCache(4, hkv, group, 1, 1, 2, codebook=CODEBOOK_ID[codebook])
    cache.page_table.copy_(torch.tensor([[1]], dtype=torch.int32))
    cache.seq_lens.fill_(320 + n)
    ok.oscar_kv_fill_history(cache.dims, rot.struct, cache.struct(), 0, 0, n, bits_tensor(bits),
                             bits_tensor(bits[::-1].copy()))
    torch.cuda.synchronize()
    exp = expected_block(bits[:, 0], bits[::-1, 0].copy(), rk[0], rv[0], ck[0], cv[0], group, n, codebook)
    assert np.array_equal(cache.pages[1, 0].cpu().numpy(), exp)
    assert not cache.pages[0].cpu().numpy().any()


@pytest.mark.parametrize("codebook", ["uniform", "lloyd-max"])
@pytest.mark.parametrize("group", [32, 64, 128])
def test_read_history_equals_oracle_dequantization(group, codebook):
    """oscar_kv_read_history returns the oracle's dequantized values bit for
    bit (R a signed permutation, so the codes themselves are exact): float32
    code * scale + zero, or the float64 Lloyd-Max value rounded once."""
    rng = np.random.default_rng(70 + group)
    B, hkv, n = 1, 2, 150
    cache = PagedKVCache(4, hkv, group, B, 3, 4, codebook=CODEBOOK_ID[codebook])
    cache.page_table.copy_(torch.tensor([[2, 0, 3]], dtype=torch.int32))
    cache.seq_lens.fill_(320 + n)
    rk, rv, ck, cv = make_rot("signed_perm", hkv, rng)
    rot = Rotation(rk, rv, ck, cv)
    kb, vb = random_tokens(rng, n, hkv), random_tokens(rng, n, hkv)
    ok.oscar_kv_fill_history(cache.dims, rot.struct, cache.struct(), 0, 0, n, bits_tensor(kb), bits_tensor(vb))
    a, m = 17, 120                                    # an unaligned range across pages
    ko = torch.full((m, hkv, 128), float("nan"), dtype=torch.float32, device="cuda")
    vo = torch.full_like(ko, float("nan"))
    ok.oscar_kv_read_history(cache.dims, cache.struct(), 0, a, m, ko, vo)
    torch.cuda.synchronize()
    ko, vo = ko.cpu().numpy(), vo.cpu().numpy()
    for j in range(hkv):
        for bits, r, c, got in ((kb, rk[j], ck[j], ko), (vb, rv[j], cv[j], vo)):
            codes, s, z = O.demote(bits[a:a + m, j], r, c, group, codebook)
            exp = O.dequantize_any(codes, s, z, group, codebook).astype(np.float32)
            assert np.array_equal(got[:, j], exp), f"kvh={j}"


@pytest.mark.parametrize("group,codebook", [(64, "uniform"), (128, "lloyd-max")])
def test_demote_keeps_other_slots_of_reused_pages(group, codebook):
    """Demotion into pages that hold stale bytes (pages reused from an
    earlier request): each step writes exactly its own slot (its key words,
    its two bits in every value word, its scale/zero entries) and leaves
    every other bit as it was, across value-word boundaries."""
    rng = np.random.default_rng(23 + group)
    hkv, hq, L0, steps = 2, 4, 330, 30   # history indices 10 .. 39 are demoted
    total = L0 + steps
    k_all = random_tokens(rng, total, hkv).reshape(total, hkv, 128)
    v_all = random_tokens(rng, total, hkv).reshape(total, hkv, 128)
    rk, rv, ck, cv = make_rot("signed_perm", hkv, rng)
    rot = Rotation(rk, rv, ck, cv)
    cache = PagedKVCache(hq, hkv, group, 1, 2, 4, codebook=CODEBOOK_ID[codebook])
    pt = np.array([[3, 1]], dtype=np.int32)
    cache.page_table.copy_(torch.from_numpy(pt))
    stale = rng.integers(0, 256, size=tuple(cache.pages.shape), dtype=np.uint8)
    cache.pages.copy_(torch.from_numpy(stale))
    cache.recent_k[0] = bits_tensor(np.stack([ring_expect(L0, k_all[:, j]) for j in range(hkv)]))
    cache.recent_v[0] = bits_tensor(np.stack([ring_expect(L0, v_all[:, j]) for j in range(hkv)]))
    L = L0
    for _ in range(steps):
        L += 1
        cache.seq_lens.fill_(L)
        ok.oscar_kv_demote(cache.dims, rot.struct, cache.struct(), bits_tensor(k_all[L - 1][None]),
                           bits_tensor(v_all[L - 1][None]))
    torch.cuda.synchronize()
    got = cache.pages.cpu().numpy()
    j0, j1 = L0 + 1 - 321, L - 321 + 1          # demoted history indices [j0, j1)
    ng = 128 // group
    for j in range(hkv):
        sl = slice(64 + j0, 64 + j1)              # their positions
        codes_k = np.zeros((64, 128), np.uint8)
        codes_v = np.zeros((64, 128), np.uint8)
        sk, zk, sv, zv = (np.zeros((64, ng), np.float32) for _ in range(4))
        codes_k[j0:j1], sk[j0:j1], zk[j0:j1] = O.demote(k_all[sl, j], rk[j], ck[j], group, codebook)
        codes_v[j0:j1], sv[j0:j1], zv[j0:j1] = O.demote(v_all[sl, j], rv[j], cv[j], group, codebook)
        new = O.pack_block(codes_k, sk, zk, codes_v, sv, zv, group)
        mask = slot_bits(slice(j0, j1), group)   # code bits of the slots
        exp = stale[pt[0, 0], j].copy()
        exp[:4096] = (exp[:4096] & ~mask[:4096]) | (new[:4096] & mask[:4096])
        for t in range(j0, j1):                  # scale/zero entries of the slots
            for half in range(2):
                a = 4096 + half * 64 * ng * 4 + O.qk_order(t) * ng * 4
                exp[a:a + ng * 4] = new[a:a + ng * 4]
        assert np.array_equal(got[pt[0, 0], j], exp), f"kvh={j}"
        assert np.array_equal(got[pt[0, 1], j], stale[pt[0, 1], j]), f"kvh={j}: untouched page changed"
        others = np.ones(got.shape[0], bool)
        others[pt[0]] = False
        assert np.array_equal(got[others], stale[others])
