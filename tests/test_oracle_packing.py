"""The oracle's packed-record writer, pinned by unpacking every code from the layout rules.

The unpacker here reads one bit pair / nibble at a time through np.unpackbits,
a different route from the packer's vectorised shifts."""
import numpy as np
import pytest

from oracle import loopkv_oracle as O
from tests.test_oracle_pins import _row


def _bits(arr_u8):
    return np.unpackbits(np.asarray(arr_u8, dtype=np.uint8), bitorder="little")


def _field(bits, pos, width):
    return sum(int(bits[pos + i]) << i for i in range(width))


def _unpack_k(buf, D, width):
    """Column-major K plane: column w of 32/width channels, 16 tokens of 32 bits each."""
    bits = _bits(buf)
    per_col = 32 // width
    out = np.zeros((16, D), dtype=np.int64)
    for t in range(16):
        for d in range(D):
            w, r = divmod(d, per_col)
            out[t, d] = _field(bits, 32 * (16 * w + t) + width * r, width)
    return out


def _stored_word(logical, n_words, r):
    """Where logical word n of a V plane is stored: quads of four words are transposed, so the
    quad q = r a + i of a plane of Q quads sits at quad position i (Q / r) + a."""
    q, k = divmod(logical, 4)
    a, i = divmod(q, r)
    return 4 * (i * (n_words // 4 // r) + a) + k


def _unpack_channel_major_2bit(buf, D):
    bits = _bits(buf)
    return np.array([[_field(bits, 32 * _stored_word(d, D, 2) + 8 * (t % 4) + 2 * (t // 4), 2) for d in range(D)]
                     for t in range(16)])


def _unpack_channel_major_4bit(buf, D):
    bits = _bits(buf)
    r = 4 if D == 256 else 2
    out = np.zeros((16, D), dtype=np.int64)
    for t in range(16):
        w, tp = divmod(t, 8)
        for d in range(D):
            out[t, d] = _field(bits, 32 * _stored_word(2 * d + w, 2 * D, r) + 8 * (tp % 4) + 4 * (tp // 4), 4)
    return out


def test_v_quads_transposed_positions():
    """The transposition on a small plane, written out: with 8 quads and r = 2 the stored order
    is quads 0, 2, 4, 6, 1, 3, 5, 7; with r = 4, quads 0, 4, 1, 5, 2, 6, 3, 7."""
    pos2 = [_stored_word(4 * q, 32, 2) // 4 for q in range(8)]
    assert [pos2.index(p) for p in range(8)] == [0, 2, 4, 6, 1, 3, 5, 7]
    pos4 = [_stored_word(4 * q, 32, 4) // 4 for q in range(8)]
    assert [pos4.index(p) for p in range(8)] == [0, 4, 1, 5, 2, 6, 3, 7]
    words = np.arange(32, dtype=np.uint64)
    assert O._transpose_quads(words, 2).reshape(8, 4)[:, 0].tolist() == [0, 8, 16, 24, 4, 12, 20, 28]


def _meta(buf):
    w = np.asarray(buf, dtype=np.uint8).view("<u4")
    s = (w & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)
    z = (w >> 16).astype(np.uint16).view(np.float16).astype(np.float64)
    return s, z


@pytest.mark.parametrize("group", [32, 64])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("layout,bits", [(O.LAYOUT_PLANES, 4), (O.LAYOUT_PLANES, 2), (O.LAYOUT_KIVI4, 4)])
def test_pack_roundtrip(D, layout, bits, group):
    rng = np.random.default_rng(D + bits + layout + group)
    q, K, V = _row(rng, 128, D, outliers=3)
    qh = O.quantize_history(K, V, bits, group)
    M = 64 * D // group   # bytes of K meta, and of V meta, in one record
    per = group // 16     # records per group
    for j in range(8):
        rec = O.pack_block(qh, j, layout)
        kind = O.KIND_Q4 if bits == 4 else O.KIND_Q2
        size = O.record_bytes(D, kind, layout, group)
        assert size % 256 == 0 and rec.size <= size < rec.size + 256
        t0 = 16 * j
        g, part = divmod(j, per)
        if layout == O.LAYOUT_KIVI4:
            kc = _unpack_k(rec[:8 * D], D, 4)
            km = rec[8 * D:8 * D + M]
            vc = _unpack_channel_major_4bit(rec[8 * D + M:16 * D + M], D)
            vm = rec[16 * D + M:16 * D + 2 * M]
            assert rec.size == 16 * D + 2 * M
        elif bits == 2:
            kc = _unpack_k(rec[:4 * D], D, 2)
            km = rec[4 * D:4 * D + M]
            vc = _unpack_channel_major_2bit(rec[4 * D + M:8 * D + M], D)
            vm = rec[8 * D + M:8 * D + 2 * M]
            assert rec.size == 8 * D + 2 * M
        else:
            kc = 4 * _unpack_k(rec[:4 * D], D, 2) + _unpack_k(rec[8 * D + 2 * M:12 * D + 2 * M], D, 2)
            vc = 4 * _unpack_channel_major_2bit(rec[4 * D + M:8 * D + M], D) + \
                _unpack_channel_major_2bit(rec[12 * D + 2 * M:16 * D + 2 * M], D)
            km, vm = rec[4 * D:4 * D + M], rec[8 * D + M:8 * D + 2 * M]
            assert rec.size == 16 * D + 2 * M
        assert np.array_equal(kc, qh["kc"][t0:t0 + 16])
        assert np.array_equal(vc, qh["vc"][t0:t0 + 16])
        ks, kz = _meta(km)
        assert ks.size == D // per
        # position -> channel inside a K column: 2-bit word byte k / bit pair p, or byte k / nibble n
        for i in range(D // per):
            pos = part * D // per + i
            if layout == O.LAYOUT_KIVI4:
                w, r = divmod(pos, 8)
                chn = 8 * w + 2 * (r % 4) + r // 4
            else:
                w, r = divmod(pos, 16)
                chn = 16 * w + 4 * (r % 4) + r // 4
            assert ks[i] == qh["ks"][g, chn] and kz[i] == qh["kz"][g, chn]
        vs, vz = _meta(vm)
        assert np.array_equal(vs.reshape(D // group, 16).T, qh["vs"][t0:t0 + 16])
        assert np.array_equal(vz.reshape(D // group, 16).T, qh["vz"][t0:t0 + 16])


def _pending_by_appends(K_bits, V_bits, group):
    """Token-by-token append model: each token enters the pending buffer at slot t mod group; when
    a group's last token arrives the group leaves for the quantizer and the buffer empties.
    Returns (position of the first pending token, pending K, pending V) after all N tokens."""
    pend_k, pend_v, first = [], [], 0
    for t in range(K_bits.shape[0]):
        assert len(pend_k) == t % group          # the slot a token takes is its position mod group
        pend_k.append(K_bits[t])
        pend_v.append(V_bits[t])
        if len(pend_k) == group:
            pend_k, pend_v, first = [], [], t + 1
    D = K_bits.shape[1]
    mk = lambda rows: np.array(rows, dtype=K_bits.dtype).reshape(len(rows), D)
    return first, mk(pend_k), mk(pend_v)


@pytest.mark.parametrize("group", [32, 64])
def test_tail_tokens_match_token_by_token_appends(group):
    """The tail (exact bf16 tokens not yet quantized) equals what a token-by-token append leaves
    pending, for lengths around group boundaries; it is shorter than a group, empty exactly at
    multiples of it, and together with the quantized prefix covers the history."""
    rng = np.random.default_rng(3)
    D = group
    for N in [0, 1, group - 1, group, group + 1, 2 * group - 1, 2 * group, 5 * group + 7]:
        kb = rng.integers(0, 1 << 16, size=(N, D), dtype=np.uint64).astype(np.uint16)
        vb = rng.integers(0, 1 << 16, size=(N, D), dtype=np.uint64).astype(np.uint16)
        first, tk, tv = O.tail_tokens(kb, vb, group)
        want_first, want_k, want_v = _pending_by_appends(kb, vb, group)
        assert first == want_first
        assert np.array_equal(tk, want_k) and np.array_equal(tv, want_v)
        assert len(tk) < group and (len(tk) == 0) == (N % group == 0)
        if N:
            qh = O.quantize_history(kb.astype(np.float64), vb.astype(np.float64), 4, group)
            assert qh["n_q"] == first and qh["n_q"] + len(tk) == N
