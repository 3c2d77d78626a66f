"""fp64 CPU oracle for LoopKV loop-aware decode attention.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports this module; only the
tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may use it. It shares no code, table or constant generator with the HIP path.

Source: "LoopKV: Loop-Aware KV Cache Compression for Serving Looped
Transformers" (arXiv:2611.04137), Abstract. The abstract fixes the method's
shape:

* every (loop, layer) cell picks 4-bit storage, 2-bit storage, or reuse of the
  final loop's KV of that layer (abstract, the sentence on the one-time
  offline profile);
* a decoding loop scores every key from the upper half of its 4-bit code and
  loads the lower half only for tokens whose weight in that loop is large enough
  to need the full code (abstract, the sentence on decoding);
* low-attention values are not skipped, since skipping compounds errors across
  loops (abstract, the sentence on skipping);
* KIVI-4, uniform 4-bit quantization, is the baseline (abstract, the serving
  sentence).

The abstract gives no formula. Where it is silent this module takes these
readings:

* KIVI-style asymmetric groups of 32 (64 as the wider option): K per channel
  over 32 consecutive tokens, V per token over 32 consecutive channels; zero = f16(min),
  scale = f16((max - min) / (2^b - 1)), each a single round-to-nearest-even
  from float64; code = clamp(rint((x - zero) / scale), 0, 2^b - 1) with
  float64 subtraction and division and ties to even; scale 0 gives code 0;
* a 4-bit code splits into hi = code >> 2 and lo = code & 3; a value whose
  low bits were not fetched is read at the bucket midpoint 4*hi + 3/2;
* a 2-bit cell is its own 2-bit quantizer, not the high plane of a 4-bit one;
* the last N mod 32 tokens of a history (the tail; N mod 64 with groups of 64)
  stay exact in bf16;
* a token t < n_q is selected when its coarse softmax weight, taken over the
  whole row including the tail, is at least tau; a selected token uses its
  4-bit K and V, the others their high-bit values; the final softmax runs over
  the refined scores of selected tokens and the coarse scores of the rest;
* a reuse cell (i, l) reads the cache of the final loop's cell (L-1, l) as it
  stands, with its own query and its own selection;
* softmax scale sigma is given (1/sqrt(D) by default); MHA, no mask.

All arithmetic is float64 on exactly represented inputs. Everything is written
step by step with no blocking, fusion or reordering beyond numpy's own matrix
products and reductions.

Parity pins: every function here is pinned by tests in ``tests/test_oracle_*``
(closed forms, brute force with exact rationals and 50-digit arithmetic,
invariants). The selected-set rule is additionally pinned only by its closed
forms (tau = 0, tau > 1) and brute force on tiny rows; the pages print no
worked example, so no value here is pinned by a number printed on the pages.
"""
from __future__ import annotations

import numpy as np

GROUP = 32          # tokens per K group, channels per V group (64 is the other supported size)
GROUPS = (32, 64)
BLOCK = 16          # tokens per paged block
KIND_Q4, KIND_Q2, KIND_SHARE = 0, 1, 2
LAYOUT_PLANES, LAYOUT_KIVI4 = 0, 1


# ---------------------------------------------------------------------------
# fp16 rounding (reading R4: one round-to-nearest-even from float64)
# ---------------------------------------------------------------------------
def f16_round(x):
    """Nearest-even float16 value of float64 ``x``, returned as float64.

    numpy converts float64 to float16 directly (one rounding); the tests pin
    this against exact rational rounding on values where a detour through
    float32 would round twice."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def f16_bits(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


# ---------------------------------------------------------------------------
# KIVI-style asymmetric group quantizer (readings R1-R3, R7)
# ---------------------------------------------------------------------------
def quantize_groups(x, bits):
    """Quantize along the last axis (a group of 32 values) to ``bits`` bits.

    Returns (codes int64 same shape, scale f64, zero f64) with scale/zero of
    shape x.shape[:-1]:
      zero  = f16(min x)
      scale = f16((max x - min x) / (2^bits - 1))
      code  = 0 if scale == 0 else clamp(rint((x - zero) / scale), 0, 2^bits - 1)
    The subtraction and division are single float64 operations; rint rounds
    half to even.
    """
    x = np.asarray(x, dtype=np.float64)
    levels = float((1 << bits) - 1)
    mn = x.min(axis=-1)
    mx = x.max(axis=-1)
    zero = f16_round(mn)
    scale = f16_round((mx - mn) / levels)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint((x - zero[..., None]) / scale[..., None])
    q = np.where(scale[..., None] == 0.0, 0.0, q)
    q = np.clip(q, 0.0, levels)
    return q.astype(np.int64), scale, zero


def quantize_history(K, V, bits, group=GROUP):
    """Quantize the complete groups of one (cell, sequence, head) history.

    K, V: float64 [N][D]; group G = 32 or 64 (D a multiple of G). Tokens
    t < n_q = G * floor(N / G) are quantized: K per channel over each G-token
    group, V per token over each run of G channels. Returns a dict with
      n_q, bits, group, kc [n_q][D], ks/kz [n_q/G][D], vc [n_q][D], vs/vz [n_q][D/G].
    """
    assert group in GROUPS
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    N, D = K.shape
    assert D % group == 0
    n_q = group * (N // group)
    ng = n_q // group
    # K: group over tokens, per channel -> move tokens to the last axis
    kg = K[:n_q].reshape(ng, group, D).transpose(0, 2, 1)          # [ng][D][G]
    kc, ks, kz = quantize_groups(kg, bits)
    kc = kc.transpose(0, 2, 1).reshape(n_q, D)
    # V: group over channels, per token
    vg = V[:n_q].reshape(n_q, D // group, group)                      # [n_q][D/G][G]
    vc, vs, vz = quantize_groups(vg, bits)
    vc = vc.reshape(n_q, D)
    return {"n_q": n_q, "bits": bits, "group": group, "kc": kc, "ks": ks, "kz": kz,
            "vc": vc, "vs": vs, "vz": vz}


# ---------------------------------------------------------------------------
# Dequantization (reading R6 for the high-bits-only value)
# ---------------------------------------------------------------------------
def _k_meta_per_token(qh):
    n_q = qh["n_q"]
    ks = np.repeat(qh["ks"], qh["group"], axis=0)[:n_q]
    kz = np.repeat(qh["kz"], qh["group"], axis=0)[:n_q]
    return ks, kz


def _v_meta_per_elem(qh):
    vs = np.repeat(qh["vs"], qh["group"], axis=1)
    vz = np.repeat(qh["vz"], qh["group"], axis=1)
    return vs, vz


def dequant_full(qh, which):
    """z + s * code for K (which='k') or V (which='v'), float64 [n_q][D]."""
    if which == "k":
        s, z = _k_meta_per_token(qh)
        c = qh["kc"]
    else:
        s, z = _v_meta_per_elem(qh)
        c = qh["vc"]
    return z + s * c.astype(np.float64)


def dequant_hi(qh, which):
    """z + s * (4 * (code >> 2) + 3/2): a 4-bit value read from its high 2 bits only."""
    assert qh["bits"] == 4
    if which == "k":
        s, z = _k_meta_per_token(qh)
        c = qh["kc"]
    else:
        s, z = _v_meta_per_elem(qh)
        c = qh["vc"]
    return z + s * (4.0 * (c >> 2).astype(np.float64) + 1.5)


# ---------------------------------------------------------------------------
# Decode of one row (cell, sequence, head)
# ---------------------------------------------------------------------------
def softmax_weights(scores):
    m = np.max(scores)
    e = np.exp(scores - m)
    return e / np.sum(e)


def decode_row(q, K, V, kind, tau, sm_scale, qh=None, sel_override=None, skip=False, group=GROUP):
    """One decode-attention row of the loop-aware method.

    q: [D] query; K, V: [N][D] history (bf16 values as float64); kind: 0 for a
    4-bit target, 1 for a 2-bit target, 'kivi4' for the uniform 4-bit
    baseline. Returns (o [D] float64, sel bool [n_q], phat [N] float64 or None).

    4-bit target (abstract, the decoding sentence; readings R8-R10):
      1. coarse scores  s_t = sigma * q . x_hi(K_t) for t < n_q, sigma * q . K_t on the tail;
      2. coarse softmax p_t = exp(s_t - max s) / sum_u exp(s_u - max s) over all N tokens;
      3. Sel = {t < n_q : p_t >= tau};
      4. refined scores sigma * q . x_4bit(K_t) on Sel, coarse elsewhere;
      5. values x_4bit(V_t) on Sel, x_hi(V_t) on the other quantized tokens
         (read at 2 bits, never skipped), exact on the tail;
      6. o = softmax(refined scores) . values.
    2-bit target: one pass over x_2bit K and V, no selection.

    skip=True is the rejected alternative of the abstract's sentence on skipping (the
    ablation, not the method): steps 1-4 as above, but the unselected quantized tokens are
    dropped instead of read at 2 bits, so the softmax runs over the selected tokens and the
    tail only (reading: a skipped token leaves the attention entirely, as in sparse
    attention); if nothing is kept, o = 0. 4-bit targets only.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    N, D = K.shape
    sigma = float(sm_scale)
    if N == 0:
        return np.zeros(D), np.zeros(0, dtype=bool), None
    bits = 2 if kind == KIND_Q2 else 4
    if qh is None:
        qh = quantize_history(K, V, bits, group)
    n_q = qh["n_q"]

    if kind == KIND_Q2:
        Kt = np.concatenate([dequant_full(qh, "k"), K[n_q:]])
        Vt = np.concatenate([dequant_full(qh, "v"), V[n_q:]])
        w = softmax_weights(sigma * (Kt @ q))
        return w @ Vt, np.zeros(n_q, dtype=bool), None

    k_hi = np.concatenate([dequant_hi(qh, "k"), K[n_q:]])
    coarse = sigma * (k_hi @ q)
    phat = softmax_weights(coarse)
    if kind == "kivi4":
        sel = np.ones(n_q, dtype=bool)
    elif sel_override is not None:
        sel = np.asarray(sel_override, dtype=bool)
    else:
        sel = phat[:n_q] >= tau
    k4 = dequant_full(qh, "k")
    scores = coarse.copy()
    scores[:n_q][sel] = sigma * (k4[sel] @ q)
    v_vals = np.concatenate([dequant_hi(qh, "v"), V[n_q:]])
    v4 = dequant_full(qh, "v")
    v_vals[:n_q][sel] = v4[sel]
    if skip:
        if kind != KIND_Q4:
            raise ValueError("skipping applies to 4-bit targets")
        keep = np.concatenate([sel, np.ones(N - n_q, dtype=bool)])
        if not keep.any():
            return np.zeros(D), sel, phat
        w = softmax_weights(scores[keep])
        return w @ v_vals[keep], sel, phat
    w = softmax_weights(scores)
    return w @ v_vals, sel, phat


def attention_reference(q, Kt, Vt, sm_scale):
    """Textbook softmax attention over given (dequantized) keys and values."""
    s = float(sm_scale) * (np.asarray(Kt, np.float64) @ np.asarray(q, np.float64))
    w = np.exp(s - s.max())
    return (w / w.sum()) @ np.asarray(Vt, np.float64)


# ---------------------------------------------------------------------------
# Packed record layout (bit-exact contract with the library)
# ---------------------------------------------------------------------------
def _pack_2bit_k(c):
    """[16][D] codes -> D/16 columns x 16 tokens of little-endian u32 (column-major).

    Word (w, t) holds channels 16w..16w+15 of token t: channel 16w + 4k + p at
    bit 8k + 2p. Words are ordered w-major, so a column's 16 tokens are contiguous."""
    T, D = c.shape
    cw = c.astype(np.uint64).reshape(T, D // 16, 4, 4)            # [t][w][k][p]
    shifts = (8 * np.arange(4)[:, None] + 2 * np.arange(4)[None, :]).astype(np.uint64)
    words = (cw << shifts).sum(axis=(2, 3))                        # [t][w]
    return words.T.reshape(-1).astype("<u4").view(np.uint8)


def _transpose_quads(words, r):
    """A V plane's 16-byte quads (runs of 4 words) stored transposed: logical quad q = r a + i
    goes to position i (nq / r) + a."""
    nq = words.size // 4
    return words.reshape(nq // r, r, 4).transpose(1, 0, 2).reshape(-1)


def _pack_2bit_channel_major(c):
    """[16][D] codes -> D little-endian u32, word d (logical order) holding channel d with
    token t at bit 8*(t%4) + 2*(t//4); the plane's quads are stored transposed with r = 2."""
    T, D = c.shape
    words = np.zeros(D, dtype=np.uint64)
    for t in range(T):
        words |= c[t].astype(np.uint64) << np.uint64(8 * (t % 4) + 2 * (t // 4))
    return _transpose_quads(words, 2).astype("<u4").view(np.uint8)


def _pack_4bit_k(c):
    """[16][D] codes -> D/8 columns x 16 tokens of u32 (column-major); word (w, t) holds
    channels 8w..8w+7 of token t: channel 8w + 2k + n at bit 8k + 4n."""
    T, D = c.shape
    cw = c.astype(np.uint64).reshape(T, D // 8, 4, 2)             # [t][w][k][n]
    shifts = (8 * np.arange(4)[:, None] + 4 * np.arange(2)[None, :]).astype(np.uint64)
    words = (cw << shifts).sum(axis=(2, 3))
    return words.T.reshape(-1).astype("<u4").view(np.uint8)


def _pack_4bit_channel_major(c):
    """[16][D] codes -> D*2 u32 (channel-major: logical word 2d + w covers tokens 8w..8w+7 of
    channel d, token t' = t - 8w at bit 8*(t'%4) + 4*(t'//4)); the plane's quads are stored
    transposed with r = 2 (D <= 128) or 4 (D = 256)."""
    T, D = c.shape
    words = np.zeros((D, 2), dtype=np.uint64)
    for t in range(T):
        w, tp = divmod(t, 8)
        words[:, w] |= c[t].astype(np.uint64) << np.uint64(8 * (tp % 4) + 4 * (tp // 4))
    return _transpose_quads(words.reshape(-1), 4 if D == 256 else 2).astype("<u4").view(np.uint8)


def _meta_words(s, z):
    """u32 words: float16 scale in bits 0-15, float16 zero in bits 16-31."""
    w = f16_bits(s).astype(np.uint32) | (f16_bits(z).astype(np.uint32) << np.uint32(16))
    return w.astype("<u4").view(np.uint8)


def k_meta_order(D, bits):
    """Channel stored at each K-meta position, inside every K column.

    2-bit planes: position 16w + 4p + k holds channel 16w + 4k + p (the channel at
    byte k, bit pair p of column word w). KIVI-4: position 8w + 4n + k holds channel
    8w + 2k + n (byte k, nibble n)."""
    pos = np.arange(D)
    if bits == 2:
        w, r = divmod(pos, 16)
        p, k = divmod(r, 4)
        return 16 * w + 4 * k + p
    w, r = divmod(pos, 8)
    n, k = divmod(r, 4)
    return 8 * w + 2 * k + n


def record_bytes(head_dim, kind, layout, group=GROUP):
    """Bytes of one 16-token record: codes (4-bit: 16D, 2-bit: 8D) plus K and V meta
    (64 D / group bytes each), padded to a multiple of 256."""
    D = head_dim
    codes = 8 * D if (layout == LAYOUT_PLANES and kind == KIND_Q2) else 16 * D
    n = codes + 2 * (64 * D // group)
    return (n + 255) // 256 * 256


def pack_block(qh, j, layout=LAYOUT_PLANES):
    """Bytes of the record of logical block j (tokens 16j..16j+15, all quantized).

    4-bit, planes layout: [K_hi | K_meta | V_hi | V_meta | K_lo | V_lo]
    2-bit:                [K2   | K_meta | V2   | V_meta]
    4-bit, KIVI-4 layout: [K4   | K_meta | V4   | V_meta]
    K planes are column-major (16-channel columns of the 16 tokens), V planes
    channel-major with their 16-byte quads stored transposed (see the helpers above).
    K_meta of group g = j // P (P = group / 16 blocks per group) holds one word per
    channel in the order of k_meta_order (a permutation inside each K column),
    split over the group's P blocks: block P g + i holds positions i D/P ..
    (i+1) D/P - 1. V_meta is [D/group channel groups][16 tokens]. The returned bytes
    stop before the record's padding (record_bytes rounds up to 256).
    """
    t0 = BLOCK * j
    assert t0 + BLOCK <= qh["n_q"]
    kc = qh["kc"][t0:t0 + BLOCK]
    vc = qh["vc"][t0:t0 + BLOCK]
    D = kc.shape[1]
    per = qh["group"] // BLOCK
    g, part = divmod(j, per)
    order = k_meta_order(D, 4 if layout == LAYOUT_KIVI4 else 2)
    ch = order[part * D // per:(part + 1) * D // per]
    kmeta = _meta_words(qh["ks"][g, ch], qh["kz"][g, ch])
    vmeta = _meta_words(qh["vs"][t0:t0 + BLOCK].T.reshape(-1), qh["vz"][t0:t0 + BLOCK].T.reshape(-1))
    if layout == LAYOUT_KIVI4:
        parts = [_pack_4bit_k(kc), kmeta, _pack_4bit_channel_major(vc), vmeta]
    elif qh["bits"] == 2:
        parts = [_pack_2bit_k(kc), kmeta, _pack_2bit_channel_major(vc), vmeta]
    else:
        parts = [_pack_2bit_k(kc >> 2), kmeta, _pack_2bit_channel_major(vc >> 2), vmeta,
                 _pack_2bit_k(kc & 3), _pack_2bit_channel_major(vc & 3)]
    return np.concatenate(parts)


def tail_tokens(K_bits, V_bits, group=GROUP):
    """Tail of a history given as bf16 bit patterns [N][D]: the last N mod group tokens,
    returned as (first position, K bits, V bits). Slot of position t is t mod group."""
    N = K_bits.shape[0]
    n_q = group * (N // group)
    return n_q, K_bits[n_q:], V_bits[n_q:]


# ---------------------------------------------------------------------------
# Whole plan helpers
# ---------------------------------------------------------------------------
def storage_cell(plan, cell):
    """Reading R13: a reuse cell (i, l) reads the final loop's cell (L-1, l)."""
    plan = np.asarray(plan)
    n_loops, n_layers = plan.shape
    if plan.reshape(-1)[cell] == KIND_SHARE:
        return (n_loops - 1) * n_layers + cell % n_layers
    return cell


def target_kind(plan, cell):
    """Kind of the cache a cell reads (a reuse cell reads its final-loop cell's kind)."""
    plan = np.asarray(plan)
    return int(plan.reshape(-1)[storage_cell(plan, cell)])
