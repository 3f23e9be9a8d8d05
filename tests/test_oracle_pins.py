"""Pins of the CPU oracle to facts other than itself.

Each ``pin_*`` function takes an oracle instance and raises AssertionError if
the oracle disagrees with what the pages print, with the mathematics (closed
forms, invariants, brute force), or with a library routine (numpy's binary16
conversion, numpy float64 matmul). The ``test_*`` wrappers run them on the
real oracle; ``test_planted_mistakes_are_caught`` compiles copies of the
oracle with one deliberate mistake each and checks that some pin fails.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle as oracle_pkg
from oracle import Oracle, Q4_0, Q8_0, Q4_K, Q6_K

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
MIB = 1024.0 * 1024.0


@pytest.fixture(scope="module")
def orc():
    return oracle_pkg.default()


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ fp16 --

def pin_f16_decode_all(orc: Oracle):
    h = np.arange(65536, dtype=np.uint16)
    got = orc.f16_to_f64_array(h)
    ref = h.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zero
    assert math.copysign(1.0, got[0x8000]) == -1.0


def pin_f16_encode_sweep(orc: Oracle):
    # every finite half, every midpoint between neighbouring halves (ties),
    # the quarter points, and random float32 bit patterns over all exponents.
    h = np.arange(0, 0x7C00, dtype=np.uint16)
    v = h.view(np.float16).astype(np.float64)
    nxt = np.append(v[1:], 65520.0)  # 65520 = the overflow threshold of 65504
    mids = (v + nxt) / 2
    quarter = v + (nxt - v) / 4
    three_q = v + 3 * (nxt - v) / 4
    pos = np.concatenate([v, mids, quarter, three_q]).astype(np.float32)
    rng = np.random.default_rng(1234)
    # about 10^7 values in all
    rand_bits = rng.integers(0, 2**32, size=6_500_000, dtype=np.uint64).astype(np.uint32)
    rand = rand_bits.view(np.float32)
    near = (rng.uniform(-27, 17, size=3_000_000)).astype(np.float64)
    near = (np.exp2(near) * rng.choice([-1.0, 1.0], size=near.size)).astype(np.float32)
    allv = np.concatenate([pos, -pos, rand, near])
    got = orc.f32_to_f16_array(allv)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = allv.astype(np.float16).view(np.uint16)
    nan = np.isnan(allv)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x3FF) != 0)


def test_f16_decode_all_halves(orc):
    pin_f16_decode_all(orc)


def test_f16_encode_matches_numpy(orc):
    pin_f16_encode_sweep(orc)


# ----------------------------------------------------------- block sizes --

def pin_block_sizes(orc: Oracle):
    facts = _golden("page_facts.json")
    q4 = facts["q4_0_block"]
    assert orc.block_elems(Q4_0) == q4["weights"]
    assert orc.block_bytes(Q4_0) == q4["bytes"]
    bpw = 8.0 * orc.block_bytes(Q4_0) / orc.block_elems(Q4_0)
    assert bpw == q4["bits_per_weight"]
    assert round(16 / bpw, 1) == q4["ratio_vs_fp16"]
    assert round(32 / bpw, 1) == q4["ratio_vs_fp32"]
    q8bpw = 8.0 * orc.block_bytes(Q8_0) / orc.block_elems(Q8_0)
    assert round(q8bpw, 1) == facts["legacy_bits_per_weight"]["q8_0_about"]
    ks = facts["kquant_superblock"]
    assert orc.block_elems(Q4_K) == ks["weights"] == ks["sub_blocks"] * ks["sub_block_weights"]
    assert orc.block_elems(Q6_K) == ks["weights"]
    # the quantizers emit exactly these sizes
    for f in (Q4_0, Q8_0, Q4_K, Q6_K):
        be, bb = orc.block_elems(f), orc.block_bytes(f)
        out = orc.quantize(f, np.zeros((3, 2 * be), np.float32))
        assert out.shape == (3, 2 * bb)
    kv = facts["kv_bytes_per_element"]
    assert round(orc.block_bytes(Q8_0) / 32, 2) == kv["q8_0_about"]
    assert round(orc.block_bytes(Q4_0) / 32, 2) == kv["q4_0"]


def _qwen3_tensors():
    """(name, rows, K) of the Qwen3-0.6B weight matrices, from the metadata the
    page prints (28 blocks, 16 q heads / 8 kv heads of 128, hidden 1024) and
    FFN width 3072; the embedding is 1024 x 151936 and tied to the output."""
    facts = _golden("page_facts.json")
    md = facts["qwen3_0p6b_metadata"]
    voc = facts["qwen3_0p6b_vocab_and_embedding"]
    hid, hd = voc["hidden"], md["key_length"]
    q, kv, ffn = md["head_count"] * hd, md["head_count_kv"] * hd, 3072
    layer = [("attn_q", q, hid), ("attn_k", kv, hid), ("attn_v", kv, hid),
             ("attn_output", hid, q), ("ffn_gate", ffn, hid), ("ffn_up", ffn, hid),
             ("ffn_down", hid, ffn)]
    mats = [(f"blk.{l}.{n}", r, k) for l in range(md["block_count"]) for (n, r, k) in layer]
    emb = ("token_embd", voc["vocab"], hid)
    norms = md["block_count"] * (hid + hid + hd + hd) + hid  # 4 per layer + output
    n_norm_tensors = 4 * md["block_count"] + 1
    return mats, emb, norms, n_norm_tensors


def pin_qwen3_file_sizes(orc: Oracle):
    facts = _golden("page_facts.json")
    sizes = facts["qwen3_0p6b_file_sizes"]
    types = facts["qwen3_0p6b_q4_k_m_tensor_types"]
    mats, emb, norm_elems, n_norm = _qwen3_tensors()
    assert n_norm == types["f32"]
    assert len(mats) + 1 == types["q4_K"] + types["q6_K"]
    n_weights = sum(r * k for _, r, k in mats) + emb[1] * emb[2]
    n_params = n_weights + norm_elems

    def q_bytes(fmt, r, k):
        return r * orc.row_bytes(fmt, k)

    # Q8_0 file: every matrix in Q8_0, norms f32
    q8 = sum(q_bytes(Q8_0, r, k) for _, r, k in mats) + q_bytes(Q8_0, emb[1], emb[2]) + 4 * norm_elems
    assert round(q8 / MIB, 2) == sizes["q8_0_mib"]
    assert round(8.0 * q8 / n_params, 2) == sizes["q8_0_bpw"]

    # q6_K block size implied by the 121.71 MiB embedding (256 weights/block)
    emb_mib = facts["qwen3_0p6b_vocab_and_embedding"]["embedding_q6_K_mib"]
    q6_bytes = round(emb_mib * MIB / (emb[1] * emb[2] / 256))
    assert q6_bytes == 210 == orc.block_bytes(Q6_K)
    assert round(emb[1] * orc.row_bytes(Q6_K, emb[2]) / MIB, 2) == emb_mib

    # Q4_K_M file: embedding + 28 of the layer matrices in q6_K (attn_v and
    # ffn_down, split a/28-a), the rest in Q4_K; only a = 14 reproduces the
    # printed size, and only with a 144-byte Q4_K block.
    matches = []
    for a in range(0, 29):
        v_up = {f"blk.{l}.attn_v" for l in range(a)}
        d_up = {f"blk.{l}.ffn_down" for l in range(28 - a)}
        tot = emb[1] * emb[2] // 256 * q6_bytes + 4 * norm_elems
        n6 = 1
        for name, r, k in mats:
            if name in v_up or name in d_up:
                tot += r * k // 256 * q6_bytes
                n6 += 1
            else:
                tot += q_bytes(Q4_K, r, k)
        if round(tot / MIB, 2) == sizes["q4_k_m_mib"] and n6 == types["q6_K"]:
            matches.append((a, round(8.0 * tot / n_params, 2)))
    assert matches == [(14, sizes["q4_k_m_bpw"])]

    # KV cache: 28 layers x (K,V) x 8 heads x 128 x 2 B = 112 KiB per token
    kvf = facts["qwen3_0p6b_kv_cache"]
    md = facts["qwen3_0p6b_metadata"]
    per_tok = md["block_count"] * 2 * md["head_count_kv"] * md["key_length"] * 2
    assert per_tok == md["kv_kib_per_token_f16"] * 1024
    assert per_tok * kvf["cells"] / MIB == kvf["f16_total_mib"]
    # q8_0 cache: same element count at block_bytes/32 bytes per element
    q8_total = per_tok / 2 * kvf["cells"] * orc.block_bytes(Q8_0) / 32
    assert q8_total / MIB == kvf["q8_0_total_mib"]
    assert q8_total / 2 / MIB == kvf["q8_0_k_mib"]


def test_block_sizes_match_pages(orc):
    pin_block_sizes(orc)


def test_qwen3_file_sizes_match_pages(orc):
    pin_qwen3_file_sizes(orc)


# ------------------------------------------------------- golden blocks --

def pin_golden_blocks(orc: Oracle):
    g = _golden("blocks.json")
    for name, fmt in (("q4_0", Q4_0), ("q8_0", Q8_0)):
        blk = np.frombuffer(bytes.fromhex(g[name]["hex"]), dtype=np.uint8)
        vals = np.array(g[name]["values"], dtype=np.float64)
        deq = orc.dequant(fmt, blk, 1, 32)[0]
        assert np.array_equal(deq, vals), name
        q = orc.quantize(fmt, vals.astype(np.float32)[None, :])[0]
        assert np.array_equal(q, blk), name


def _q4k_handmade():
    """A Q4_K superblock written from the layout text: d = 2^-6, dmin = 2^-7,
    sub-block scales/mins chosen so that max sc = max mn = 63, codes with low
    nibble t and high nibble 15-t. Returns (bytes, values)."""
    d, dmin = 2.0 ** -6, 2.0 ** -7
    sc = [63, 1, 17, 32, 5, 40, 8, 63]
    mn = [0, 63, 10, 1, 33, 7, 63, 20]
    V = 0
    for f, v in enumerate(sc + mn):
        V |= v << (6 * f)
    hdr = np.float16(d).tobytes() + np.float16(dmin).tobytes() + V.to_bytes(12, "little")
    codes = bytes((t | ((15 - t) << 4)) for _ in range(8) for t in range(16))
    vals = np.empty(256)
    for j in range(8):
        for t in range(16):
            vals[32 * j + t] = d * sc[j] * t - dmin * mn[j]
            vals[32 * j + 16 + t] = d * sc[j] * (15 - t) - dmin * mn[j]
    return np.frombuffer(hdr + codes, dtype=np.uint8), vals


def pin_q4k_layout(orc: Oracle):
    blk, vals = _q4k_handmade()
    assert blk.size == orc.block_bytes(Q4_K)
    assert np.array_equal(orc.dequant(Q4_K, blk, 1, 256)[0], vals)
    assert np.array_equal(orc.quantize(Q4_K, vals.astype(np.float32)[None, :])[0], blk)


def _q6k_pack(d, sc, codes):
    """Q6_K-style superblock bytes written from the layout text: fp16 d, then
    per 32-weight group g: int8 scales of sub-blocks 2g and 2g+1, 16 bytes
    with code 32g+t's low 4 bits in the low nibble of byte t and code
    32g+16+t's in the high nibble, then little-endian words H0, H1 whose byte
    b holds the high 2 bits of codes 32g+4w+b (H0) or 32g+16+4w+b (H1) at
    bits 2w..2w+1."""
    out = bytearray(np.float16(d).tobytes())
    for g in range(8):
        c = codes[32 * g:32 * g + 32]
        out += bytes([sc[2 * g] & 0xFF, sc[2 * g + 1] & 0xFF])
        out += bytes((c[t] & 15) | ((c[16 + t] & 15) << 4) for t in range(16))
        for half in (0, 16):
            h = 0
            for w in range(4):
                for b in range(4):
                    h |= (c[half + 4 * w + b] >> 4) << (8 * b + 2 * w)
            out += h.to_bytes(4, "little")
    return np.frombuffer(bytes(out), dtype=np.uint8)


def _q6k_handmade():
    """A Q6_K superblock: d = 2^-8, sub-block scales with maximum 127, codes
    in 1..63 with one code of magnitude 31 per sub-block (so quantizing the
    values must give back exactly these bytes). Returns (bytes, values)."""
    d = 2.0 ** -8
    sc = [127, 1, 64, 33, 5, 127, 90, 12, 7, 100, 45, 3, 127, 60, 2, 77]
    codes = [1 + (7 * e + 11 * (e // 16) + 3) % 63 for e in range(256)]
    for j in range(16):
        codes[16 * j + (j % 16)] = 63 if j % 2 == 0 else 1
    vals = np.array([d * sc[e // 16] * (codes[e] - 32) for e in range(256)])
    return _q6k_pack(d, sc, codes), vals


def pin_q6k_layout(orc: Oracle):
    blk, vals = _q6k_handmade()
    assert blk.size == orc.block_bytes(Q6_K)
    assert np.array_equal(orc.dequant(Q6_K, blk, 1, 256)[0], vals)
    assert np.array_equal(orc.quantize(Q6_K, vals.astype(np.float32)[None, :])[0], blk)


def test_golden_blocks(orc):
    pin_golden_blocks(orc)


def test_q6k_layout(orc):
    pin_q6k_layout(orc)


def test_q4k_layout(orc):
    pin_q4k_layout(orc)


# --------------------------------------------------------- quantizer math --

def _test_blocks(rng, nblk, be):
    """A mix of block populations: N(0, 0.02) with outliers, N(0, 1), a heavy
    tail, tiny (fp16 subnormal) scales, all-equal, all-negative blocks."""
    parts = [
        rng.normal(0, 0.02, (nblk, be)),
        rng.normal(0, 1.0, (nblk, be)),
        rng.standard_t(2, (nblk, be)) * 0.01,
        rng.normal(0, 1e-6, (nblk // 4, be)),
        rng.normal(0, 1e-9, (nblk // 4, be)),
        np.full((nblk // 8, be), 0.0375),
        -np.abs(rng.normal(0, 0.5, (nblk // 4, be))),
        np.abs(rng.normal(0, 0.5, (nblk // 4, be))),
    ]
    W = np.concatenate(parts).astype(np.float32)
    out = W.reshape(-1, be).copy()
    # outliers in 5% of the first population's blocks
    idx = rng.choice(nblk, size=nblk // 20, replace=False)
    out[idx, rng.integers(0, be, idx.size)] = 0.2 * rng.choice([-1, 1], idx.size)
    return out


def _scales_q40_q80(blocks: np.ndarray, orc: Oracle, fmt) -> np.ndarray:
    h = blocks[:, 0].astype(np.uint16) | (blocks[:, 1].astype(np.uint16) << 8)
    return orc.f16_to_f64_array(h)


def pin_round_trip_bound(orc: Oracle):
    rng = np.random.default_rng(7)
    for fmt in (Q4_0, Q8_0):
        W = _test_blocks(rng, 4000, 32)
        B = orc.quantize(fmt, W)
        Wd = orc.dequant(fmt, B, W.shape[0], 32)
        D = _scales_q40_q80(B, orc, fmt)
        err = np.abs(Wd - W.astype(np.float64))
        # The bound scale/2 holds where the fp16 scale is a normal number
        # (relative rounding <= 2^-11 keeps every |w|/D within the code range).
        normal = D >= 2.0 ** -14
        assert np.all(err[normal] <= D[normal, None] / 2 * (1 + 1e-6)), fmt
        # and the bound is reached (not vacuous): some error above 0.45 D
        assert np.any(err[normal] > 0.45 * D[normal, None])
        # D == 0 only when amax/qmax rounds to zero in fp16 (below 2^-25)
        qmax = 7 if fmt == Q4_0 else 127
        zero = D == 0
        assert np.all(np.abs(W[zero]) <= qmax * 2.0 ** -25) and np.all(Wd[zero] == 0)
        # subnormal scales: the worst case is clamping at the largest code
        sub = ~normal & ~zero
        assert np.all(err[sub] <= np.maximum(D[sub, None] / 2,
                                             np.abs(W[sub]).max(axis=1, keepdims=True) - qmax * D[sub, None]) * (1 + 1e-6))
    # Q4_K: within [-O_j, 15 S_j - O_j] the error is at most S_j/2; outside,
    # the value is clamped to the nearer end.
    W = _test_blocks(rng, 500, 256)
    B = orc.quantize(Q4_K, W)
    Wd = orc.dequant(Q4_K, B, W.shape[0], 256)
    S, O = _q4k_scales(B, orc)
    w = W.astype(np.float64).reshape(-1, 8, 32)
    wd = Wd.reshape(-1, 8, 32)
    lo, hi = -O[..., None], (15 * S - O)[..., None]
    inside = (w >= lo) & (w <= hi)
    err = np.abs(wd - w)
    assert np.all(err[inside] <= (np.broadcast_to(S[..., None], w.shape)[inside] / 2) * (1 + 1e-6) + 1e-300)
    dist = np.where(w < lo, lo - w, w - hi)
    assert np.allclose(err[~inside], dist[~inside], rtol=1e-12, atol=0)
    # Q6_K: within [-32 S_j, 31 S_j] the error is at most S_j/2, reached;
    # outside, clamped to the nearer end
    W = _test_blocks(rng, 500, 256)
    B = orc.quantize(Q6_K, W)
    Wd = orc.dequant(Q6_K, B, W.shape[0], 256).reshape(-1, 16, 16)
    S, _ = _q6k_fields(B, orc)
    w = W.astype(np.float64).reshape(-1, 16, 16)
    lo, hi = -32 * S[..., None], 31 * S[..., None]
    inside = (w >= lo) & (w <= hi)
    err = np.abs(Wd - w)
    Sb = np.broadcast_to(S[..., None], w.shape)
    assert np.all(err[inside] <= Sb[inside] / 2 * (1 + 1e-6) + 1e-300)
    assert np.any(err[inside] > 0.45 * Sb[inside])
    dist = np.where(w < lo, lo - w, w - hi)
    assert np.allclose(err[~inside], dist[~inside], rtol=1e-12, atol=0)


def _q4k_scales(B: np.ndarray, orc: Oracle):
    d = orc.f16_to_f64_array(B[:, 0].astype(np.uint16) | (B[:, 1].astype(np.uint16) << 8))
    dm = orc.f16_to_f64_array(B[:, 2].astype(np.uint16) | (B[:, 3].astype(np.uint16) << 8))
    V = [int.from_bytes(bytes(row[4:16]), "little") for row in B]
    sc = np.array([[(v >> (6 * j)) & 63 for j in range(8)] for v in V], dtype=np.float64)
    mn = np.array([[(v >> (6 * (8 + j))) & 63 for j in range(8)] for v in V], dtype=np.float64)
    return d[:, None] * sc, dm[:, None] * mn


def _q6k_fields(B: np.ndarray, orc: Oracle):
    """Per superblock: the 16 sub-block scales S_j = d*sc_j (fp64) and the 256
    codes (0..63), read with the layout of _q6k_pack."""
    d = orc.f16_to_f64_array(B[:, 0].astype(np.uint16) | (B[:, 1].astype(np.uint16) << 8))
    G = B[:, 2:].reshape(-1, 8, 26)
    sc = G[:, :, 0:2].view(np.int8).astype(np.float64).reshape(-1, 16)
    nib = G[:, :, 2:18].astype(np.int64)
    lo = np.concatenate([nib & 15, nib >> 4], axis=2)            # [n, 8, 32]
    H = G[:, :, 18:26].astype(np.int64).reshape(-1, 8, 2, 4)      # [n, g, half, byte b]
    e = np.arange(16)
    hi = (H[:, :, :, e & 3] >> (2 * (e >> 2))) & 3              # [n, g, half, 16]
    codes = lo + 16 * hi.reshape(-1, 8, 32)
    return d[:, None] * sc, codes.reshape(-1, 256)


def _codes_q40(B):
    c = B[:, 2:18]
    return np.concatenate([c & 15, c >> 4], axis=1).astype(np.int64) - 8


def _codes_q80(B):
    return B[:, 2:34].view(np.int8).astype(np.int64)


def pin_code_optimality(orc: Oracle):
    """Every code is the nearest grid point to its weight (brute force over
    all codes); exact ties go away from zero."""
    rng = np.random.default_rng(11)
    for fmt, codes_of, grid in ((Q4_0, _codes_q40, np.arange(-8, 8)),
                                (Q8_0, _codes_q80, np.arange(-127, 128))):
        W = _test_blocks(rng, 1500, 32)
        B = orc.quantize(fmt, W)
        D = _scales_q40_q80(B, orc, fmt)
        q = codes_of(B)
        w = W.astype(np.float64)
        ok = D > 0
        cand = D[ok, None, None] * grid[None, None, :]
        errs = np.abs(w[ok][..., None] - cand)
        best = errs.min(axis=-1)
        chosen = np.abs(w[ok] - D[ok, None] * q[ok])
        assert np.all(chosen <= best + 1e-6 * D[ok, None])
        assert np.all(q[~ok] == 0)
    # exact ties: 1.25 / 0.5 = 2.5 -> 3 (half away from zero), -1.25 -> -3
    x = np.zeros(32, np.float32)
    x[0], x[1], x[2], x[3] = 3.5, 1.25, -1.25, 0.25
    q = _codes_q40(orc.quantize(Q4_0, x[None, :]))[0]
    assert (q[1], q[2], q[3]) == (3, -3, 1)
    # Q4_K codes: nearest of the 16 levels S*q - O to each weight
    W = _test_blocks(rng, 300, 256)
    B = orc.quantize(Q4_K, W)
    S, O = _q4k_scales(B, orc)
    c = B[:, 16:].reshape(-1, 8, 16)
    qk = np.concatenate([c & 15, c >> 4], axis=2).astype(np.float64)
    w = W.astype(np.float64).reshape(-1, 8, 32)
    lv = S[..., None, None] * np.arange(16)[None, None, None, :] - O[..., None, None]
    best = np.abs(w[..., None] - lv).min(axis=-1)
    chosen = np.abs(w - (S[..., None] * qk - O[..., None]))
    assert np.all(chosen <= best + 1e-6 * S[..., None])
    # Q6_K codes: nearest of the 64 levels S_j (c - 32)
    W = _test_blocks(rng, 300, 256)
    B = orc.quantize(Q6_K, W)
    S, c = _q6k_fields(B, orc)
    w = W.astype(np.float64).reshape(-1, 16, 16)
    q = c.reshape(-1, 16, 16).astype(np.float64) - 32
    lv = S[..., None, None] * (np.arange(64) - 32)[None, None, None, :]
    best = np.abs(w[..., None] - lv).min(axis=-1)
    chosen = np.abs(w - S[..., None] * q)
    assert np.all(chosen <= best + 1e-6 * S[..., None])
    # a zero scale gives the zero code
    assert np.all(c.reshape(-1, 16, 16)[S == 0] == 32)


def pin_idempotence(orc: Oracle):
    rng = np.random.default_rng(5)
    for fmt in (Q4_0, Q8_0):
        W = _test_blocks(rng, 3000, 32)
        B = orc.quantize(fmt, W)
        Wd = orc.dequant(fmt, B, W.shape[0], 32).astype(np.float32)
        # Proof: the largest |code| of a block with a normal fp16 scale is
        # exactly qmax, so amax' = qmax*D, d' = D and every code repeats.
        # (Subnormal scales can clamp to -8 or miss qmax; they are excluded.)
        normal = _scales_q40_q80(B, orc, fmt) >= 2.0 ** -14
        assert normal.sum() > 0.8 * normal.size
        assert np.array_equal(orc.quantize(fmt, Wd[normal]), B[normal])


def pin_exact_grid(orc: Oracle):
    """W = D*q with D an fp16 value and q on the grid (largest |q| present):
    the quantizer must return exactly D and q."""
    rng = np.random.default_rng(3)
    n = 2000
    for fmt, qmax, codes_of in ((Q4_0, 7, _codes_q40), (Q8_0, 127, _codes_q80)):
        # D: random binary16 values, normal and subnormal, small enough that
        # qmax*D stays finite in fp16 range
        hb = rng.integers(1, 0x5800 if qmax == 7 else 0x5000, n).astype(np.uint16)
        D = hb.view(np.float16).astype(np.float64)
        q = rng.integers(-qmax, qmax + 1, (n, 32))
        q[np.arange(n), rng.integers(0, 32, n)] = qmax * rng.choice([-1, 1], n)
        W = (D[:, None] * q).astype(np.float32)
        assert np.array_equal(W.astype(np.float64), D[:, None] * q)
        B = orc.quantize(fmt, W)
        assert np.array_equal(_scales_q40_q80(B, orc, fmt), D)
        assert np.array_equal(codes_of(B), q)


def pin_q6k_exact_grid(orc: Oracle):
    """Random superblocks on the Q6_K grid (d a normal binary16 value,
    largest scale 127, every non-zero sub-block holding a code of magnitude
    31; some sub-blocks all zero): quantizing their values returns exactly
    the bytes _q6k_pack writes for them."""
    rng = np.random.default_rng(13)
    for _ in range(200):
        d = float(np.uint16(rng.integers(0x0800, 0x3800)).view(np.float16))
        sc = rng.integers(1, 128, 16)
        sc[rng.integers(0, 16)] = 127
        codes = rng.integers(1, 64, 256)
        for j in range(16):
            codes[16 * j + rng.integers(0, 16)] = rng.choice([1, 63])
        zero = rng.random(16) < 0.15
        zero[np.argmax(sc)] = False
        for j in np.flatnonzero(zero):
            sc[j] = 0
            codes[16 * j:16 * j + 16] = 32
        vals = np.array([d * sc[e // 16] * (codes[e] - 32) for e in range(256)])
        assert np.array_equal(vals.astype(np.float32).astype(np.float64), vals)
        blk = _q6k_pack(d, [int(v) for v in sc], [int(v) for v in codes])
        assert np.array_equal(orc.quantize(Q6_K, vals.astype(np.float32)[None, :])[0], blk)
        assert np.array_equal(orc.dequant(Q6_K, blk, 1, 256)[0], vals)


def pin_zero_blocks(orc: Oracle):
    Z = np.zeros((2, 256), np.float32)
    b4 = orc.quantize(Q4_0, Z)
    assert np.all(b4.reshape(-1, 18)[:, :2] == 0) and np.all(b4.reshape(-1, 18)[:, 2:] == 0x88)
    b8 = orc.quantize(Q8_0, Z)
    assert np.all(b8 == 0)
    bk = orc.quantize(Q4_K, Z)
    assert np.all(bk == 0)
    b6 = orc.quantize(Q6_K, Z)
    assert np.array_equal(b6[0], _q6k_pack(0.0, [0] * 16, [32] * 256))
    for f in (Q4_0, Q8_0, Q4_K, Q6_K):
        assert np.all(orc.dequant(f, orc.quantize(f, Z), 2, 256) == 0)


def test_round_trip_bound(orc):
    pin_round_trip_bound(orc)


def test_code_optimality(orc):
    pin_code_optimality(orc)


def test_idempotence(orc):
    pin_idempotence(orc)


def test_exact_grid(orc):
    pin_exact_grid(orc)


def test_zero_blocks(orc):
    pin_zero_blocks(orc)


def test_q6k_exact_grid(orc):
    pin_q6k_exact_grid(orc)


# ----------------------------------------------------------------- matmul --

def pin_gemv_special_cases(orc: Oracle):
    rng = np.random.default_rng(21)
    M, K = 6, 512
    for fmt in (Q4_0, Q8_0, Q4_K, Q6_K):
        W = rng.normal(0, 0.02, (M, K)).astype(np.float32)
        B = orc.quantize(fmt, W)
        Wd = orc.dequant(fmt, B, M, K)
        for k in (0, 1, 17, 255, K - 1):
            x = np.zeros(K, np.float32)
            x[k] = 1.0
            assert np.array_equal(orc.gemv(fmt, B, x, M, K), Wd[:, k])
        ones = np.ones(K, np.float32)
        assert np.allclose(orc.gemv(fmt, B, ones, M, K), Wd.sum(axis=1), rtol=1e-13, atol=0)


def pin_brute_force_4x64(orc: Oracle):
    """4x64 products by a pure-Python triple loop on the dequantized values,
    and by numpy float64 matmul."""
    rng = np.random.default_rng(64)
    M, K, N = 4, 64, 3
    x = rng.normal(0, 1, K).astype(np.float32)
    X = rng.normal(0, 1, (N, K)).astype(np.float32)
    Xq = orc.quantize(Q8_0, X)
    Xd = orc.dequant(Q8_0, Xq, N, K)
    for fmt in (Q4_0, Q8_0):
        W = rng.normal(0, 0.02, (M, K)).astype(np.float32)
        B = orc.quantize(fmt, W)
        Wd = orc.dequant(fmt, B, M, K).tolist()
        y = orc.gemv(fmt, B, x, M, K)
        Y = orc.gemm(fmt, B, Xq, M, K, N)
        for m in range(M):
            s = 0.0
            for k in range(K):
                s += Wd[m][k] * float(x[k])
            assert y[m] == s
            for n in range(N):
                s = 0.0
                for k in range(K):
                    s += Wd[m][k] * float(Xd[n][k])
                assert Y[n][m] == s
        assert np.allclose(y, np.array(Wd) @ x.astype(np.float64), rtol=1e-14, atol=1e-15)
        assert np.allclose(Y, Xd @ np.array(Wd).T, rtol=1e-14, atol=1e-15)
    # the superblock formats on one 256-wide row pair, against the values
    # the layout text gives for a hand-built superblock
    blk, vals = _q6k_handmade()
    B = np.concatenate([blk, blk[::-1].copy()])[None, :].reshape(1, -1)
    K = 512
    Wd = orc.dequant(Q6_K, B, 1, K)[0]
    assert np.array_equal(Wd[:256], vals)
    x = rng.normal(0, 1, K).astype(np.float32)
    X = rng.normal(0, 1, (2, K)).astype(np.float32)
    Xq = orc.quantize(Q8_0, X)
    Xd = orc.dequant(Q8_0, Xq, 2, K)
    s = 0.0
    for k in range(K):
        s += float(Wd[k]) * float(x[k])
    assert orc.gemv(Q6_K, B, x, 1, K)[0] == s
    Y = orc.gemm(Q6_K, B, Xq, 1, K, 2)
    for n in range(2):
        s = 0.0
        for k in range(K):
            s += float(Wd[k]) * float(Xd[n][k])
        assert Y[n][0] == s


def pin_on_grid_products(orc: Oracle):
    """On-grid fp32 matrices quantize losslessly, so the oracle's products
    must equal numpy's float64 products of the raw inputs (no dequant code
    involved on the reference side)."""
    rng = np.random.default_rng(99)
    M, K, N = 9, 320, 5
    D = np.ldexp(1.0, rng.integers(-9, -4, (M, K // 32)))
    q = rng.integers(-7, 8, (M, K // 32, 32))
    q[:, :, 0] = 7
    W = (D[..., None] * q).reshape(M, K).astype(np.float32)
    x = rng.normal(0, 1, K).astype(np.float32)
    y = orc.gemv(Q4_0, orc.quantize(Q4_0, W), x, M, K)
    assert np.allclose(y, W.astype(np.float64) @ x.astype(np.float64), rtol=1e-13, atol=1e-15)
    Dx = np.ldexp(1.0, rng.integers(-7, -3, (N, K // 32)))
    qx = rng.integers(-127, 128, (N, K // 32, 32))
    qx[:, :, 5] = -127
    X = (Dx[..., None] * qx).reshape(N, K).astype(np.float32)
    Y = orc.gemm(Q4_0, orc.quantize(Q4_0, W), orc.quantize(Q8_0, X), M, K, N)
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    assert np.allclose(Y, ref, rtol=1e-13, atol=1e-15)


def test_gemv_special_cases(orc):
    pin_gemv_special_cases(orc)


def test_brute_force_4x64(orc):
    pin_brute_force_4x64(orc)


def test_on_grid_products(orc):
    pin_on_grid_products(orc)


# ------------------------------------------------------------ KV cache --

def _q4_0_pack(D, q):
    """Q4_0 blocks from the layout text (fp16 scale, byte t = code t | code
    t+16 << 4, code = q + 8) for scales D [nblk] and integers q [nblk][32]."""
    out = bytearray()
    for d, qq in zip(D, q):
        c = [int(v) + 8 for v in qq]
        out += np.float16(d).tobytes() + bytes(c[t] | (c[t + 16] << 4) for t in range(16))
    return np.frombuffer(bytes(out), dtype=np.uint8)


def pin_kv_write(orc: Oracle):
    """KV rows written as Q4_0/Q8_0 blocks at their cells, minus the
    per-channel bias when one is given; other cells untouched."""
    rng = np.random.default_rng(31)
    dim, cells, n, cell0 = 256, 9, 4, 3
    # rows = bias + D q exactly, |q| = 7 present in every block: centred, the
    # quantizer must return exactly D and q (lpnh.cn KV-cache article, section
    # kv-mean-center 进阶技巧: subtract the fixed bias before Q4_0 quantization)
    bias = rng.integers(-128, 129, dim) * 2.0 ** -4
    D = 2.0 ** -rng.integers(5, 9, (n, dim // 32))
    q = rng.integers(-7, 8, (n, dim // 32, 32))
    q[:, :, 0] = 7 * rng.choice([-1, 1], (n, dim // 32))
    rows = (bias.reshape(1, -1) + (D[..., None] * q).reshape(n, dim))
    assert np.array_equal(rows.astype(np.float32).astype(np.float64), rows)
    cache = rng.integers(0, 256, (cells, orc.row_bytes(Q4_0, dim)), dtype=np.uint8)
    out = orc.kv_write(Q4_0, rows.astype(np.float32), bias.astype(np.float32), cache, cell0)
    want = _q4_0_pack(D.reshape(-1), q.reshape(-1, 32)).reshape(n, -1)
    assert np.array_equal(out[cell0:cell0 + n], want)
    keep = np.r_[0:cell0, cell0 + n:cells]
    assert np.array_equal(out[keep], cache[keep])
    # without a bias the rows are quantized as they are
    for fmt in (Q4_0, Q8_0):
        c0 = np.zeros((cells, orc.row_bytes(fmt, dim)), np.uint8)
        o2 = orc.kv_write(fmt, rows.astype(np.float32), None, c0, 0)
        assert np.array_equal(orc.dequant(fmt, o2[:n], n, dim),
                              orc.dequant(fmt, orc.quantize(fmt, rows.astype(np.float32)), n, dim))
    # shapes and formats outside the contract are refused
    for bad in (lambda: orc.kv_write(Q4_K, np.zeros((1, 256), np.float32), None,
                                     np.zeros((2, orc.row_bytes(Q4_K, 256)), np.uint8), 0),
                lambda: orc.kv_write(Q8_0, np.zeros((2, 64), np.float32), None,
                                     np.zeros((2, orc.row_bytes(Q8_0, 64)), np.uint8), 1)):
        with pytest.raises(ValueError):
            bad()


def pin_kv_mean_center(orc: Oracle):
    """The article's argument for the bias: a query's scores against the
    centred keys differ from the raw ones by the same constant q.k_mean for
    every key, and softmax ignores a constant added to a row; and centring
    channels with a large mean shrinks the Q4_0 error."""
    rng = np.random.default_rng(41)
    nk, dim = 50, 128
    mean = rng.normal(0, 4, dim)
    K = (mean + rng.normal(0, 0.3, (nk, dim))).astype(np.float32)
    qv = rng.normal(0, 1, (7, dim))
    def softmax(z):
        z = z - z.max(axis=1, keepdims=True)
        e = np.exp(z)
        return e / e.sum(axis=1, keepdims=True)
    s_raw = qv @ K.astype(np.float64).T
    s_cen = qv @ (K.astype(np.float64) - mean).T
    assert np.allclose(s_raw - s_cen, (qv @ mean)[:, None], rtol=1e-12, atol=1e-9)
    assert np.allclose(softmax(s_raw), softmax(s_cen), rtol=1e-10, atol=1e-15)
    bias = mean.astype(np.float32)
    c = np.zeros((nk, orc.row_bytes(Q4_0, dim)), np.uint8)
    raw = orc.dequant(Q4_0, orc.kv_write(Q4_0, K, None, c, 0), nk, dim)
    cen = orc.dequant(Q4_0, orc.kv_write(Q4_0, K, bias, c, 0), nk, dim) + bias
    e_raw = np.linalg.norm(raw - K)
    e_cen = np.linalg.norm(cen - K)
    assert e_cen < e_raw / 5, (e_cen, e_raw)


def test_kv_write(orc):
    pin_kv_write(orc)


def test_kv_mean_center(orc):
    pin_kv_mean_center(orc)


# ---------------------------------------------------------- planted mistakes

ALL_PINS = [pin_f16_decode_all, pin_f16_encode_sweep, pin_block_sizes,
            pin_qwen3_file_sizes, pin_golden_blocks, pin_q4k_layout,
            pin_q6k_layout, pin_round_trip_bound, pin_code_optimality,
            pin_idempotence, pin_exact_grid, pin_q6k_exact_grid, pin_zero_blocks,
            pin_gemv_special_cases, pin_brute_force_4x64, pin_on_grid_products,
            pin_kv_write, pin_kv_mean_center]

MUTANTS = {
    "nibble_order_swapped": ("blk[2 + t] = (uint8_t)(code[t] | (code[t + 16] << 4));",
                             "blk[2 + t] = (uint8_t)(code[t + 16] | (code[t] << 4));"),
    "q4_0_offset_7": ("w[t] = D * (double)(lo - 8);", "w[t] = D * (double)(lo - 7);"),
    "q4_0_scale_over_8": ("float d = amax / 7.0f;", "float d = amax / 8.0f;"),
    "q8_0_scale_over_128": ("float d = amax / 127.0f;", "float d = amax / 128.0f;"),
    "codes_from_unrounded_scale": (
        "float q = clampf(rnd(x[i] / D), -8.0f, 7.0f);",
        "float q = clampf(rnd(x[i] / d), -8.0f, 7.0f);"),
    "round_half_even": ("static float rnd(float t) { return roundf(t); }",
                        "static float rnd(float t) { return rintf(t); }"),
    "f16_ties_up": ("n = whole + ((rem > half || (rem == half && (whole & 1u))) ? 1u : 0u);",
                    "n = whole + ((rem >= half) ? 1u : 0u);"),
    "f16_no_subnormals": ("int q = (e < -14 ? -14 : e) - 10;", "int q = e - 10;"),
    "scale_byte_order": ("dst[0] = (uint8_t)(h & 0xFFu);\n  dst[1] = (uint8_t)(h >> 8);",
                         "dst[1] = (uint8_t)(h & 0xFFu);\n  dst[0] = (uint8_t)(h >> 8);"),
    "q4k_min_sign": ("float O = Dm * (float)mnq[j];", "float O = -Dm * (float)mnq[j];"),
    "q4k_field_order": ("int v = f < 8 ? sc[f] : mnq[f - 8];", "int v = f < 8 ? mnq[f] : sc[f - 8];"),
    "q6k_scale_over_32": ("s[j] = amax / 31.0f;", "s[j] = amax / 32.0f;"),
    "q6k_code_offset_31": ("w[32 * g + e] = D * (double)sc * (double)(code6(grp, e) - 32);",
                           "w[32 * g + e] = D * (double)sc * (double)(code6(grp, e) - 31);"),
    "q6k_high_bits_words_swapped": ("int hi = (grp[18 + 4 * half + b] >> (2 * w)) & 3;",
                                    "int hi = (grp[22 - 4 * half + b] >> (2 * w)) & 3;"),
    "q6k_one_scale_per_group": ("memcpy(&sc, grp + (e >> 4), 1);", "memcpy(&sc, grp, 1);"),
    "kv_bias_added": ("x[e] = bias ? v - bias[b * 32 + e] : v;", "x[e] = bias ? v + bias[b * 32 + e] : v;"),
    "kv_cell_offset_ignored": ("uint8_t *blk = cache + ((cell0 + i) * nb + b) * bb;",
                               "uint8_t *blk = cache + (i * nb + b) * bb;"),
    "gemv_drops_last_element": ("for (int64_t k = 0; k < K; ++k) s += w[k] * (double)x[k];",
                                "for (int64_t k = 0; k + 1 < K; ++k) s += w[k] * (double)x[k];"),
    "gemm_transposed_store": ("Y[n * M + m] = s;", "Y[(m * N + n) % (M * N)] = s;"),
    "gemm_x_block_stride_32": (
        "dequant_block(ORC_Q8_0, Xq8 + (n * nbx + b) * 34, X + n * K + b * 32);",
        "dequant_block(ORC_Q8_0, Xq8 + (n * nbx + b) * 32, X + n * K + b * 32);"),
}


@pytest.mark.slow
def test_planted_mistakes_are_caught(tmp_path):
    src = open(oracle_pkg.SRC).read()
    survivors = []
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) == 1, f"mutation anchor for {name} not unique"
        path = tmp_path / f"{name}.c"
        path.write_text(src.replace(old, new))
        lib = oracle_pkg.compile_c(str(path), str(tmp_path / f"lib{name}.so"))
        mut = Oracle(lib)
        caught = False
        for pin in ALL_PINS:
            try:
                pin(mut)
            except (AssertionError, ValueError):
                caught = True
                break
        if not caught:
            survivors.append(name)
    assert survivors == []
