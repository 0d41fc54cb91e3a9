"""Pins for the oracle's masked and variable-length forward (fso_forward_masked).

Masks come before the score shift and probability generation ("Fused
softmax makes quantized attention faster on AMD GPUs", section "What the
evidence shows"): a masked key takes no part in any tile maximum (reference
or gate) and its P is 0.  Causal masks align the queries to the end of the
keys: query i sees key k when k <= i + kv_len - q_len.

Pins, each chosen so that a plausible mistake in the mask logic fails one:
  * brute force on tiny inputs against the independent exact-rational forward
    (tests/spec_numpy.py) given each row's visible prefix: P codes, scales and
    counts bit-exact, O to 1e-12 (causal with Sq = Skv, Sq < Skv and Sq > Skv,
    per-batch q_lens / kv_lens, planted rollbacks);
  * key padding reduces to the shorter problem: kv_len = L on Skv keys (V rows
    >= L zero) equals the unmasked problem on the first L keys, bit for bit;
  * causal row i equals the unmasked one-query problem on keys
    [0, i + Skv - Sq] with the same quantized K and V;
  * closed form: with Sq = Skv, causal row 0 sees only key 0, so P = 1, l = 1
    and O is V-hat row 0;
  * rows past q_len and rows with no visible key are 0 with count 0;
  * a mask that hides nothing equals the unmasked forward.
"""
import math

import numpy as np
import pytest
import torch

from tests import spec_numpy as spec
from tests.test_oracle_forward import bits, quantize_all, rand_bf16


def visible_counts(Sq, Skv, causal, q_len=None, kv_len=None):
    """keys seen by each query row of one batch (the definition above)"""
    ql = Sq if q_len is None else max(0, min(Sq, q_len))
    kl = Skv if kv_len is None else max(0, min(Skv, kv_len))
    out = np.zeros(Sq, np.int64)
    for i in range(ql):
        n = kl
        if causal:
            n = min(n, i + kl - ql + 1)
        out[i] = max(n, 0)
    return out


BRUTE = [
    # (name, Sq, Skv, D, qk, v, p, kv_tile, causal, q_len, kv_len, stressed key rows)
    ("causal-square", 40, 100, 32, 2, 2, 2, 32, True, 40, 40, None),
    ("causal-sq<skv", 6, 130, 32, 2, 2, 2, 64, True, None, None, (20, 90, 120)),
    ("causal-sq>skv", 70, 33, 32, 4, 4, 2, 32, True, None, None, None),
    ("kvlen-fp8", 5, 160, 32, 0, 0, 0, 64, False, None, 97, (66, 70, 80, 90, 96, 101)),
    ("qlen-kvlen-causal", 9, 96, 64, 2, 2, 2, 32, True, 7, 61, None),
]


@pytest.mark.parametrize("case", BRUTE, ids=[c[0] for c in BRUTE])
def test_masked_matches_exact_spec(oracle, case):
    name, Sq, Skv, D, qk, ve, pe, bc, causal, q_len, kv_len, stress = case
    seed = sum(map(ord, name)) % 997
    q = rand_bf16((1, 1, Sq, D), seed)
    k = rand_bf16((1, 1, Skv, D), seed + 1)
    v = rand_bf16((1, 1, Skv, D), seed + 2)
    if stress:
        k = k.float()
        for r in stress:
            k[0, 0, r] *= 8.0
        k = k.to(torch.bfloat16)
    sigma = 1 / math.sqrt(D)
    Q, K, V = quantize_all(oracle, q, k, v, sigma, qk, ve)
    p = oracle.make_params(1, 1, Sq, Skv, D, qk, ve, pe, tau=8.0, kv_tile=bc)
    ql = None if q_len is None else [q_len]
    kl = None if kv_len is None else [kv_len]
    r = oracle.forward(p, Q, K, V, want_p=True, causal=causal, q_lens=ql, kv_lens=kl)
    vis = visible_counts(Sq, Skv, causal, q_len, kv_len)
    O_s, cnt_s, pc_s, ps_s = spec.forward(bits(q[0, 0]), bits(k[0, 0]), bits(v[0, 0]), sigma, qk, ve, pe,
                                          tau=8.0, kv_tile=bc, visible=vis)
    assert np.array_equal(r["counts"], cnt_s)
    assert np.array_equal(r["p_codes"].astype(np.int64), pc_s)
    assert np.array_equal(r["p_scales"].astype(np.int64), ps_s)
    np.testing.assert_allclose(r["O"], O_s, rtol=1e-12, atol=1e-12)
    if stress:
        assert r["counts"].sum() > 0, "stress case should exercise the rollback path"
    # masked rows: zero output, zero l, zero count
    dead = vis == 0
    assert np.all(r["O"][dead] == 0) and np.all(r["l"][dead] == 0) and np.all(r["counts"][dead] == 0)


@pytest.mark.parametrize("qk,ve,pe,bc", [(2, 2, 2, 64), (4, 4, 2, 128), (0, 0, 0, 64)])
def test_key_padding_is_truncation(oracle, qk, ve, pe, bc):
    """kv_lens = [L0, L1] equals, per batch, the unmasked problem on its first L keys
    (V rows >= L are zero, so V's key blocks quantize identically)."""
    B, H, Sq, Skv, D = 2, 2, 20, 300, 64
    lens = [137, 64]
    q = rand_bf16((B, H, Sq, D), 11)
    k = rand_bf16((B, H, Skv, D), 12, scale=4.0)
    v = rand_bf16((B, H, Skv, D), 13)
    v = v.clone()
    for b, L in enumerate(lens):
        v[b, :, L:] = 0
    sigma = 1 / math.sqrt(D)
    Q, K, V = quantize_all(oracle, q, k, v, sigma, qk, ve)
    p = oracle.make_params(B, H, Sq, Skv, D, qk, ve, pe, tau=1.0, kv_tile=bc)
    r = oracle.forward(p, Q, K, V, want_p=True, kv_lens=lens)
    for b, L in enumerate(lens):
        Qb, Kb, Vb = quantize_all(oracle, q[b:b + 1], k[b:b + 1, :, :L].contiguous(), v[b:b + 1, :, :L].contiguous(),
                                  sigma, qk, ve)
        pb = oracle.make_params(1, H, Sq, L, D, qk, ve, pe, tau=1.0, kv_tile=bc)
        rb = oracle.forward(pb, Qb, Kb, Vb, want_p=True)
        sl = slice(b * H * Sq, (b + 1) * H * Sq)
        assert np.array_equal(r["O"][sl], rb["O"])
        assert np.array_equal(r["l"][sl], rb["l"])
        assert np.array_equal(r["counts"][sl], rb["counts"])
        s32 = rb["p_codes"].shape[1]
        assert np.array_equal(r["p_codes"][sl, :s32], rb["p_codes"])
        assert not r["p_codes"][sl, s32:].any()
        assert np.array_equal(r["p_scales"][sl, :s32 // 32], rb["p_scales"])
    assert r["counts"].sum() > 0


@pytest.mark.parametrize("Sq,Skv", [(48, 48), (30, 130), (90, 40)])
def test_causal_row_is_prefix_problem(oracle, Sq, Skv):
    """causal row i equals the one-query problem on keys [0, i + Skv - Sq] fed the
    same quantized K rows and the first V key blocks of each feature."""
    H, D, qk, ve, pe, bc = 1, 64, 2, 2, 2, 32
    q = rand_bf16((1, H, Sq, D), 21)
    k = rand_bf16((1, H, Skv, D), 22, scale=2.0)
    v = rand_bf16((1, H, Skv, D), 23)
    sigma = 1 / math.sqrt(D)
    Q, K, V = quantize_all(oracle, q, k, v, sigma, qk, ve)
    p = oracle.make_params(1, H, Sq, Skv, D, qk, ve, pe, tau=4.0, kv_tile=bc)
    r = oracle.forward(p, Q, K, V, want_p=True, causal=True)
    qbb, vbb = oracle.block_bytes(qk), oracle.block_bytes(ve)
    nbd = D // 32
    nb32 = (Skv + 31) // 32
    qc = Q[0].reshape(Sq, nbd, qbb)
    qs = Q[1].reshape(Sq, nbd)
    kc = K[0].reshape(Skv, nbd, kbb := qbb)
    ks = K[1].reshape(Skv, nbd)
    vc = V[0].reshape(D, nb32, vbb)
    vs = V[1].reshape(D, nb32)
    for i in range(Sq):
        n = i + Skv - Sq + 1
        if n <= 0:
            assert not r["O"][i].any() and r["l"][i] == 0 and r["counts"][i] == 0
            continue
        n = min(n, Skv)
        nb = (n + 31) // 32
        pi = oracle.make_params(1, 1, 1, n, D, qk, ve, pe, tau=4.0, kv_tile=bc)
        ri = oracle.forward(pi, (qc[i:i + 1].copy(), qs[i:i + 1].copy()), (kc[:n].copy(), ks[:n].copy()),
                            (vc[:, :nb].copy(), vs[:, :nb].copy()), want_p=True)
        assert np.array_equal(r["O"][i], ri["O"][0]), i
        assert r["l"][i] == ri["l"][0] and r["counts"][i] == ri["counts"][0]
        assert np.array_equal(r["p_codes"][i, :32 * nb], ri["p_codes"][0])
        assert not r["p_codes"][i, 32 * nb:].any()


@pytest.mark.parametrize("pe", [0, 2])
def test_causal_first_row_closed_form(oracle, pe):
    """Sq = Skv, causal: row 0 sees key 0 alone; its folded score lands on T0,
    stage 1 gives the BF16 pattern of 1.0, P-hat = 1 and O = V-hat row 0."""
    S, D = 64, 64
    q = rand_bf16((1, 1, S, D), 31)
    k = rand_bf16((1, 1, S, D), 32)
    v = rand_bf16((1, 1, S, D), 33)
    sigma = 1 / math.sqrt(D)
    Q, K, V = quantize_all(oracle, q, k, v, sigma, 2, 2)
    p = oracle.make_params(1, 1, S, S, D, 2, 2, pe, tau=8.0, kv_tile=64)
    r = oracle.forward(p, Q, K, V, want_p=True, causal=True)
    vbb = oracle.block_bytes(2)
    vc = V[0].reshape(D, 2, vbb)
    vs = V[1].reshape(D, 2)
    # V-hat row 0 from the oracle's own codec on the code bytes: element 0 of
    # block 0 of each feature (6-bit little-endian stream: low 6 bits of byte 0)
    v0 = np.array([oracle.decode(2, int(vc[d, 0, 0]) & 0x3F) * 2.0 ** (int(vs[d, 0]) - 127) for d in range(D)])
    assert r["l"][0] == 1.0
    assert np.array_equal(r["O"][0], v0)
    assert r["p_codes"][0, 1:].sum() == 0


def test_qlen_rows_zero_and_full_mask_is_identity(oracle):
    B, H, Sq, Skv, D = 2, 1, 30, 70, 32
    q = rand_bf16((B, H, Sq, D), 41)
    k = rand_bf16((B, H, Skv, D), 42)
    v = rand_bf16((B, H, Skv, D), 43)
    sigma = 1 / math.sqrt(D)
    Q, K, V = quantize_all(oracle, q, k, v, sigma, 2, 2)
    p = oracle.make_params(B, H, Sq, Skv, D, 2, 2, 2, tau=8.0, kv_tile=64)
    base = oracle.forward(p, Q, K, V, want_p=True)
    same = oracle.forward(p, Q, K, V, want_p=True, q_lens=[Sq, Sq], kv_lens=[Skv, Skv])
    for key in ("O", "l", "counts", "p_codes", "p_scales"):
        assert np.array_equal(base[key], same[key])
    r = oracle.forward(p, Q, K, V, q_lens=[12, 0], kv_lens=[Skv, 0])
    O = r["O"].reshape(B, Sq, D)
    assert np.array_equal(O[0, :12], base["O"].reshape(B, Sq, D)[0, :12])
    assert not O[0, 12:].any() and not O[1].any()
    # one query, causal, aligned to the end of the keys: it sees every key
    p1 = oracle.make_params(1, 1, 1, Skv, D, 2, 2, 2, tau=8.0, kv_tile=64)
    Q1 = (Q[0].reshape(B, Sq, -1)[0, -1:].copy(), Q[1].reshape(B, Sq, -1)[0, -1:].copy())
    K1 = (K[0].reshape(B, -1)[0].copy(), K[1].reshape(B, -1)[0].copy())
    V1 = (V[0].reshape(B, -1)[0].copy(), V[1].reshape(B, -1)[0].copy())
    a = oracle.forward(p1, Q1, K1, V1)
    c = oracle.forward(p1, Q1, K1, V1, causal=True)
    assert np.array_equal(a["O"], c["O"])


@pytest.mark.parametrize("Sq,Skv", [(40, 40), (25, 90), (60, 30)])
def test_masked_r0_is_prefix_softmax(oracle, Sq, Skv):
    """R0 under a causal mask and key lengths: row i equals the unmasked R0 of
    the one-query problem on its visible keys; rows that see nothing are 0."""
    B, H, D = 2, 1, 32
    q = bits(rand_bf16((B, H, Sq, D), 51))
    k = bits(rand_bf16((B, H, Skv, D), 52))
    v = bits(rand_bf16((B, H, Skv, D), 53))
    kv_lens = [Skv, max(1, Skv // 2)]
    q_lens = [Sq, Sq - 3]
    sigma = 0.2
    R = oracle.reference_bf16(q, k, v, sigma, causal=True, q_lens=q_lens, kv_lens=kv_lens)
    for b in range(B):
        vis = visible_counts(Sq, Skv, True, q_lens[b], kv_lens[b])
        for i in range(Sq):
            row = R[b * Sq + i]
            if vis[i] == 0:
                assert not row.any()
                continue
            n = int(vis[i])
            ref = oracle.reference_bf16(q[b:b + 1, :, i:i + 1].copy(), k[b:b + 1, :, :n].copy(),
                                        v[b:b + 1, :, :n].copy(), sigma)
            assert np.array_equal(row, ref[0]), (b, i)
