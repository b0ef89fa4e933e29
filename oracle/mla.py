"""fp64 NumPy oracle: naive and weight-absorbed MLA decode over a latent cache.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it and
for the citation tags [AUDIT], [MLA80], [TRACE]).

All arithmetic is float64 on the exact values of the bf16 inputs (``dtype`` may
be lowered to float32 only to reproduce the pages' fp32-level gap between the
two association orders, [AUDIT] §5.3 and [MLA80] §4). Nothing here rounds an
intermediate to bf16.

Notation (per sequence; one attention layer):

* ``c_kv[t]``  512-dim shared KV latent of key token t          ([AUDIT] §2.1)
* ``k_pe[t]``  64-dim decoupled RoPE key, shared by all heads    ([AUDIT] §2.4, [MLA80] §2)
* ``q_nope[i,h]`` 128-dim content query, ``q_pe[i,h]`` 64-dim rope query
* ``w_uk[h]``, ``w_uv[h]``  per-head up-projections, shape [128, 512]: the
  per-head slices of the ``nn.Linear(d_c, n_h*d_h)`` weights of [MLA80] §2
  (the ``Wuk``/``Wuv`` rows of head h), so ``k_c = w_uk[h] @ c_kv[t]``.

Query i of a sequence with ``L`` keys (keys include this step's new tokens:
the cache is concatenated before attending, [MLA80] §2 ``forward``) sits at
absolute position ``L - Lq + i`` and sees keys ``t <= L - Lq + i``.
"""

from __future__ import annotations

import math

import numpy as np

D_C = 512       # KV latent width, [AUDIT] §2.4 / [TRACE] §1.2 "KV LoRA rank 512"
D_ROPE = 64     # decoupled RoPE key width, [TRACE] §1.2
D_NOPE = 128    # per-head content q/k width, [TRACE] §1.2
D_V = 128       # per-head value width, [TRACE] §1.2
BLOCK = 64      # paged-cache block (tokens)
ROPE_BASE = 10000.0


def default_scale(d_nope: int = D_NOPE, d_rope: int = D_ROPE) -> float:
    """Softmax scale of the naive path: SDPA's default 1/sqrt(q width) on the
    (d_nope + d_rope)-wide concatenated query ([MLA80] §2 ``forward``, which
    calls ``scaled_dot_product_attention`` without a scale)."""
    return 1.0 / math.sqrt(d_nope + d_rope)


# --------------------------------------------------------------------------
# input decoding


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# RoPE ([MLA80] appendix A: build_rope / rotate_half / apply_rope)


def rope_angles(pos, d_rope: int = D_ROPE, base: float = ROPE_BASE) -> np.ndarray:
    """theta[..., i] = pos * base**(-2i/d_rope), i = 0 .. d_rope/2-1.

    One frequency per interleaved pair; [MLA80] appendix A builds the same
    frequencies from ``arange(0, dim, 2) / dim`` and repeats each one for the
    two members of its pair."""
    i = np.arange(d_rope // 2, dtype=np.float64)
    inv_freq = np.power(float(base), -(2.0 * i) / d_rope)
    return np.multiply.outer(np.asarray(pos, dtype=np.float64), inv_freq)


def rope(x, pos, base: float = ROPE_BASE, dtype=np.float64) -> np.ndarray:
    """Rotate interleaved pairs (x[2i], x[2i+1]) of the last axis by theta_i.

    ``pos`` has the shape of ``x[..., 0]`` (or broadcasts to it). The pair
    rule follows [MLA80] appendix A: ``rotate_half`` maps (a, b) -> (-b, a)
    on each even/odd pair and ``apply_rope`` forms x*cos + rotate_half(x)*sin,
    so y[2i] = x[2i] cos - x[2i+1] sin and y[2i+1] = x[2i+1] cos + x[2i] sin.
    """
    x = np.asarray(x, dtype=dtype)
    theta = rope_angles(np.asarray(pos), x.shape[-1], base).astype(dtype)
    c, s = np.cos(theta), np.sin(theta)
    xe, xo = x[..., 0::2], x[..., 1::2]
    y = np.empty(np.broadcast_shapes(x.shape, theta.shape[:-1] + (x.shape[-1],)), dtype=dtype)
    y[..., 0::2] = xe * c - xo * s
    y[..., 1::2] = xo * c + xe * s
    return y


# --------------------------------------------------------------------------
# latent cache contents ([AUDIT] §2.4, §6.1; [TRACE] §3.1)


def cache_rows(c_kv, k_pe, pos, base: float = ROPE_BASE) -> np.ndarray:
    """Value of the 576-element cache row of each appended token:
    ``[c_kv (512) | RoPE(k_pe, pos) (64)]``.

    The pages cache the shared latent and the shared rope key side by side
    (576 = 512 + 64, [AUDIT] §2.4, [TRACE] §3.1). [MLA80] §2 caches k_R
    before rotation and rotates it at every step; rotation is linear and
    depends only on the key's own position, so storing it rotated once at
    append gives the same scores (pinned by a test)."""
    c_kv = np.asarray(c_kv, dtype=np.float64)
    k_r = rope(k_pe, np.asarray(pos), base)
    return np.concatenate([c_kv, k_r], axis=-1)


# --------------------------------------------------------------------------
# absorbed path ([AUDIT] §2.2-§2.3; [MLA80] §4-§5)


def query_positions(L: int, Lq: int) -> np.ndarray:
    """Absolute positions of the Lq newest tokens of an L-key sequence."""
    return np.arange(L - Lq, L, dtype=np.int64)


def visible(q_pos, L: int) -> np.ndarray:
    """mask[i, t] = key t is visible to query i (t <= q_pos[i])."""
    return np.arange(L)[None, :] <= np.asarray(q_pos)[:, None]


def absorb_q(q_nope, q_pe, q_pos, w_uk, base: float = ROPE_BASE, dtype=np.float64):
    """q_lat[i,h] = w_uk[h]^T q_nope[i,h]  (512) and q_r[i,h] = RoPE(q_pe[i,h], q_pos[i]).

    Moving W_UK from every cached key onto the query: q^T (W_UK c) = (W_UK^T q)^T c
    ([AUDIT] §2.2; [MLA80] §4 "Path B", which forms Q_abs with an einsum over
    the head dim). Returns (q_lat [Lq,H,512], q_r [Lq,H,64])."""
    q_nope = np.asarray(q_nope, dtype=dtype)
    w_uk = np.asarray(w_uk, dtype=dtype)
    # per head: [Lq,128] @ [128,512]
    q_lat = np.matmul(q_nope.transpose(1, 0, 2), w_uk).transpose(1, 0, 2)
    q_r = rope(q_pe, np.asarray(q_pos)[:, None], base, dtype=dtype)
    return q_lat, q_r


def latent_scores(q_lat, q_r, c_kv, k_r, scale: float, dtype=np.float64) -> np.ndarray:
    """s[i,h,t] = scale * (q_lat[i,h] . c_kv[t] + q_r[i,h] . k_r[t]).

    The content part scores against the shared latent ([MLA80] §5: Q_abs .
    c_kv^T); the rope part broadcasts the one shared k_r to every head
    ([MLA80] §5 "共享 k_r 广播到各 head")."""
    q_lat = np.asarray(q_lat, dtype=dtype)
    q_r = np.asarray(q_r, dtype=dtype)
    c_kv = np.asarray(c_kv, dtype=dtype)
    k_r = np.asarray(k_r, dtype=dtype)
    return (np.matmul(q_lat, c_kv.T) + np.matmul(q_r, k_r.T)) * dtype(scale)


def masked_softmax(s, mask) -> tuple[np.ndarray, np.ndarray]:
    """Row softmax over the last axis with invisible entries excluded.

    Returns (p, lse) with lse = log sum_t exp(s_t) over visible t (natural
    log). Rows with no visible key get p = 0 and lse = -inf."""
    s = np.where(mask, s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe)
    z = np.sum(e, axis=-1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(z > 0, e / np.where(z > 0, z, 1.0), 0.0)
        lse = np.where(z[..., 0] > 0, m_safe[..., 0] + np.log(np.where(z[..., 0] > 0, z[..., 0], 1.0)), -np.inf)
    return p, lse


def latent_attention(q_lat, q_r, c_kv, k_r, q_pos, scale: float, dtype=np.float64):
    """o_lat[i,h] = sum_t p[i,h,t] c_kv[t], p = softmax over visible t.

    The value projection moves after the weighted sum: sum p (W_UV c) =
    W_UV (sum p c) ([AUDIT] §2.3; [MLA80] §5 "ctx_latent [B,H,1,d_c]").
    Returns (o_lat [Lq,H,512], lse [Lq,H])."""
    s = latent_scores(q_lat, q_r, c_kv, k_r, scale, dtype)
    L = np.asarray(c_kv).shape[0]
    mask = visible(q_pos, L)[:, None, :]
    p, lse = masked_softmax(s, mask)
    return np.matmul(p, np.asarray(c_kv, dtype=dtype)), lse


def out_up(o_lat, w_uv, dtype=np.float64) -> np.ndarray:
    """o[i,h] = w_uv[h] @ o_lat[i,h]  ([AUDIT] §2.3: W_V applied after the sum)."""
    o_lat = np.asarray(o_lat, dtype=dtype)
    w_uv = np.asarray(w_uv, dtype=dtype)
    return np.matmul(o_lat.transpose(1, 0, 2), w_uv.transpose(0, 2, 1)).transpose(1, 0, 2)


def absorbed_decode(q_nope, q_pe, c_kv, k_pe, w_uk, w_uv, scale=None, base=ROPE_BASE,
                    dtype=np.float64) -> dict:
    """Absorbed MLA attention for one sequence: Lq newest queries over L keys.

    ``k_pe`` is the un-rotated rope key of keys 0..L-1 (positions = index).
    Returns dict(q_lat, q_r, k_r, o_lat, lse, o)."""
    if scale is None:
        scale = default_scale()
    c_kv = np.asarray(c_kv, dtype=dtype)
    L, Lq = c_kv.shape[0], np.asarray(q_nope).shape[0]
    q_pos = query_positions(L, Lq)
    k_r = rope(k_pe, np.arange(L), base, dtype=dtype)
    q_lat, q_r = absorb_q(q_nope, q_pe, q_pos, w_uk, base, dtype)
    o_lat, lse = latent_attention(q_lat, q_r, c_kv, k_r, q_pos, scale, dtype)
    o = out_up(o_lat, w_uv, dtype)
    return dict(q_lat=q_lat, q_r=q_r, k_r=k_r, o_lat=o_lat, lse=lse, o=o)


# --------------------------------------------------------------------------
# FP8 latent cache ([AUDIT] §6.1: FlashMLA's support matrix lists an FP8 KV
# cache for its MQA-mode kernels; the pages name the format but not its
# scaling). Reading taken here: the 576-element row of each token is stored
# as OCP FP8 E4M3 codes ("e4m3fn": 4 exponent bits with bias 7, 3 mantissa
# bits, no infinities, 0x7f / 0xff are NaN, largest finite 448) with one fp32
# scale per token, a power of two: the smallest 2^k with max|row| / 2^k <= 448,
# k >= -124 (1 for an all-zero row). E4M3 is a floating-point format, so a
# power-of-two scale costs no precision against max|row| / 448 (it moves the
# row's largest element into (224, 448] instead of onto 448), and code x scale
# is then exactly a bf16 value. The codes are integers, so the quantizer takes
# its decisions in float32, the precision of the kernel that writes them;
# everything after decoding is fp64 again.

FP8_MAX = 448.0
FP8_MIN_SCALE_EXP = -124   # code x 2^k stays on the bf16 grid (2^-9 x 2^-124 = 2^-133)


def e4m3_decode(codes) -> np.ndarray:
    """Exact value of E4M3 (e4m3fn) codes as float64: sign bit 7, exponent
    bits 6..3 (bias 7), mantissa bits 2..0. Exponent field 0 is subnormal,
    m/8 * 2^-6; otherwise (1 + m/8) * 2^(e-7); 0x7f and 0xff are NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_encode(u) -> np.ndarray:
    """float32 values -> E4M3 codes, rounding to the nearest representable
    value (ties to the even mantissa) and saturating at +-448.

    The grid spacing is 2^(E-3) in the binade [2^E, 2^(E+1)) for E >= -6
    and 2^-9 below 2^-6 (subnormals); dividing by that power of two is exact,
    np.rint rounds half to even, and a result that reaches the next binade is
    that binade's first value."""
    u = np.asarray(u, dtype=np.float32).astype(np.float64)
    a = np.abs(u)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))      # a = f * 2^ex, f in [0.5, 1)
    E = np.maximum(ex - 1, -6)                      # binade exponent, subnormals share -6
    quantum = np.ldexp(1.0, E - 3)
    v = np.minimum(np.rint(a / quantum) * quantum, FP8_MAX)
    # code of the (now representable) magnitude v
    _, vex = np.frexp(np.where(v > 0, v, 1.0))
    ve = vex - 1
    normal = v >= 2.0 ** -6
    e_field = np.where(normal, ve + 7, 0)
    m_field = np.where(normal, np.rint((v / np.ldexp(1.0, ve) - 1.0) * 8.0), np.rint(v / 2.0 ** -9))
    code = (e_field.astype(np.int64) << 3) | m_field.astype(np.int64)
    code = np.where(np.signbit(u), code | 0x80, code)
    code = np.where(np.isnan(u), 0x7F, code)
    return code.astype(np.uint8)


def fp8_token_scale(amax) -> np.ndarray:
    """The power of two 2^k with k = max(ceil(log2(amax / 448)), -124) for
    float32 amax > 0, and 1 for amax = 0. Exactly, with amax = f 2^e and
    448 = F 2^E (f, F in [0.5, 1); F = 0.875, E = 9): amax / 2^(e-E) =
    (f / F) 448 is at most 448 when f <= F, and twice it is above 448 (f >=
    0.5 > F / 2), so k = e - E, or e - E + 1 when f > F."""
    a = np.asarray(amax, dtype=np.float32).astype(np.float64)
    f, e = np.frexp(np.where(a > 0, a, 1.0))
    F, E = np.frexp(FP8_MAX)
    k = np.where(f <= F, e - E, e - E + 1)
    k = np.maximum(k, FP8_MIN_SCALE_EXP)
    return np.where(a > 0, np.ldexp(1.0, k), 1.0).astype(np.float32)


def quantize_rows_fp8(rows) -> tuple[np.ndarray, np.ndarray]:
    """Per-token scaled FP8 of float32 rows [..., 576]: scale = the power of
    two of ``fp8_token_scale`` (1 for an all-zero row), codes = E4M3(row /
    scale); the division by a power of two is exact in float32 down to its
    subnormals, whose values all encode to code 0 or 1 alike. Returns
    (codes uint8 [..., 576], scale float32 [...])."""
    r = np.asarray(rows, dtype=np.float32)
    amax = np.max(np.abs(r), axis=-1)
    scale = fp8_token_scale(amax)
    codes = e4m3_encode((r / scale[..., None]).astype(np.float32))
    return codes, scale


def dequantize_rows_fp8(codes, scale) -> np.ndarray:
    """Row value the FP8 cache stands for: code value times its token's scale (fp64, exact)."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]


def cache_rows_fp8(c_kv, k_pe, pos, base: float = ROPE_BASE) -> tuple[np.ndarray, np.ndarray]:
    """FP8 cache row of each appended token: the same [c_kv | RoPE(k_pe, pos)]
    as ``cache_rows`` (rotation in fp64), rounded once to float32 (the
    quantizer's input precision; the bf16 latent is exact in float32), then
    quantized per token. Returns (codes [T, 576] uint8, scale [T] float32)."""
    rows = cache_rows(c_kv, k_pe, pos, base).astype(np.float32)
    return quantize_rows_fp8(rows)


def absorbed_decode_fp8(q_nope, q_pe, codes, scale, w_uk, w_uv, softmax_scale=None,
                        base=ROPE_BASE) -> dict:
    """Absorbed MLA decode of one sequence over its FP8 cache rows (keys
    0..L-1, rows already rotated): the rows are decoded exactly and attended
    to in fp64 as in ``absorbed_decode``. Returns dict(q_lat, q_r, o_lat, lse, o)."""
    if softmax_scale is None:
        softmax_scale = default_scale()
    rows = dequantize_rows_fp8(codes, scale)
    L, Lq = rows.shape[0], np.asarray(q_nope).shape[0]
    q_pos = query_positions(L, Lq)
    q_lat, q_r = absorb_q(q_nope, q_pe, q_pos, w_uk, base)
    o_lat, lse = latent_attention(q_lat, q_r, rows[:, :D_C], rows[:, D_C:], q_pos, softmax_scale)
    return dict(q_lat=q_lat, q_r=q_r, o_lat=o_lat, lse=lse, o=out_up(o_lat, w_uv))


# --------------------------------------------------------------------------
# naive (expanding) path ([AUDIT] §2.1; [MLA80] §2 MLA.forward)


def naive_decode(q_nope, q_pe, c_kv, k_pe, w_uk, w_uv, scale=None, base=ROPE_BASE,
                 dtype=np.float64, rope_on_content: bool = False) -> dict:
    """Expand per-head keys and values from the latent, then attend.

    k[t,h] = [w_uk[h] c_kv[t] | RoPE(k_pe[t], t)] (192 wide, the rope part
    shared by all heads) and v[t,h] = w_uv[h] c_kv[t] (128 wide); the query
    is [q_nope | RoPE(q_pe, p_i)]; o = softmax(q.k * scale) v over visible
    keys ([MLA80] §2 ``forward``: k_c, v, k_r_h, cat, SDPA).

    ``rope_on_content=True`` also rotates the content key (as [MLA80] §4's
    "K_C_rope" experiment does, with RoPE over the 128-dim content key); it
    exists only as a negative control: absorption no longer holds.
    Returns dict(k, v, q, o, lse)."""
    if scale is None:
        scale = default_scale()
    c_kv = np.asarray(c_kv, dtype=dtype)
    w_uk = np.asarray(w_uk, dtype=dtype)
    w_uv = np.asarray(w_uv, dtype=dtype)
    L, Lq = c_kv.shape[0], np.asarray(q_nope).shape[0]
    H = w_uk.shape[0]
    q_pos = query_positions(L, Lq)
    k_c = np.einsum("tc,hjc->thj", c_kv, w_uk)
    if rope_on_content:
        k_c = rope(k_c, np.arange(L)[:, None], base, dtype=dtype)
    v = np.einsum("tc,hjc->thj", c_kv, w_uv)
    k_r = rope(k_pe, np.arange(L), base, dtype=dtype)
    k = np.concatenate([k_c, np.broadcast_to(k_r[:, None, :], (L, H, k_r.shape[-1]))], axis=-1)
    q_r = rope(q_pe, q_pos[:, None], base, dtype=dtype)
    q = np.concatenate([np.asarray(q_nope, dtype=dtype), q_r], axis=-1)
    s = np.einsum("ihd,thd->iht", q, k) * dtype(scale)
    p, lse = masked_softmax(s, visible(q_pos, L)[:, None, :])
    o = np.einsum("iht,thj->ihj", p, v)
    return dict(k=k, v=v, q=q, o=o, lse=lse)


# --------------------------------------------------------------------------
# one whole attention layer around the decode, and a stack of layers
# ([MLA80] §2 MLA.__init__ / forward: the projections Wdq, Wuq, Wqr, Wdkv,
# Wkr, Wo around the attention; [AUDIT] §9 item 4: error over several layers)


def linear(x, w, dtype=np.float64) -> np.ndarray:
    """nn.Linear without bias: y = x @ w.T, w stored [out, in] ([MLA80] §2)."""
    return np.matmul(np.asarray(x, dtype=dtype), np.asarray(w, dtype=dtype).T)


def layer_projections(h, lw, dtype=np.float64) -> dict:
    """The new tokens' inputs of one layer from hidden states h [Lq, d_model]
    ([MLA80] §2 forward): c_kv = Wdkv h, k_pe = Wkr h (un-rotated: RoPE is
    applied where the key is used), qz = Wdq h, q_nope = Wuq qz and
    q_pe = Wqr qz, split per head. ``lw`` maps the weight names to arrays in
    nn.Linear layout ([out, in])."""
    H = np.asarray(lw["w_uk"]).shape[0]
    Lq = np.asarray(h).shape[0]
    qz = linear(h, lw["w_dq"], dtype)
    return dict(c_kv=linear(h, lw["w_dkv"], dtype), k_pe=linear(h, lw["w_kr"], dtype), qz=qz,
                q_nope=linear(qz, lw["w_uq"], dtype).reshape(Lq, H, -1),
                q_pe=linear(qz, lw["w_qr"], dtype).reshape(Lq, H, -1))


def layer_decode(h, hist_c_kv, hist_k_pe, lw, path: str = "absorbed", dtype=np.float64) -> dict:
    """One layer for one sequence: the Lq new tokens h [Lq, d_model] follow
    hist_c_kv / hist_k_pe (the cached latents of the earlier tokens, keys
    0 .. L-Lq-1); their own latents are appended before attending, and the
    layer returns y = Wo [o_0 | ... | o_{H-1}] ([MLA80] §2: the heads'
    outputs concatenated, then Wo). ``path`` picks the absorbed or the
    expanded attention (the two definitions of the same result)."""
    pr = layer_projections(h, lw, dtype)
    c_kv = np.concatenate([np.asarray(hist_c_kv, dtype=dtype), pr["c_kv"]])
    k_pe = np.concatenate([np.asarray(hist_k_pe, dtype=dtype), pr["k_pe"]])
    if path == "absorbed":
        att = absorbed_decode(pr["q_nope"], pr["q_pe"], c_kv, k_pe, lw["w_uk"], lw["w_uv"], dtype=dtype)
    elif path == "naive":
        att = naive_decode(pr["q_nope"], pr["q_pe"], c_kv, k_pe, lw["w_uk"], lw["w_uv"], dtype=dtype)
    else:
        raise ValueError(path)
    Lq = np.asarray(h).shape[0]
    y = linear(att["o"].reshape(Lq, -1), lw["w_o"], dtype)
    return dict(pr, o=att["o"], y=y)


def stack_decode(h0, hists, layers, dtype=np.float64) -> list:
    """Layers applied in turn with a residual connection around each:
    h_{l+1} = h_l + layer_l(h_l). The residual is a reading: the pages'
    module is one layer returning Wo(o) alone, and a stack of layers adds its
    output to the stream it read. Returns [h_1, ..., h_n]."""
    h = np.asarray(h0, dtype=dtype)
    out = []
    for (hc, hk), lw in zip(hists, layers):
        h = h + layer_decode(h, hc, hk, lw, dtype=dtype)["y"]
        out.append(h)
    return out


# --------------------------------------------------------------------------
# split-KV partials and their merge (flash-decode split of the key range)


def partial_attention(q_lat, q_r, c_kv, k_r, q_pos, scale: float, t0: int, t1: int):
    """Unnormalised partial over keys [t0, t1): returns (m, l, acc) with
    m = max visible score, l = sum exp(s - m), acc = sum exp(s - m) c_kv[t].
    A range with no visible key gives m = -inf, l = 0, acc = 0."""
    s = latent_scores(q_lat, q_r, c_kv[t0:t1], k_r[t0:t1], scale)
    mask = (np.arange(t0, t1)[None, :] <= np.asarray(q_pos)[:, None])[:, None, :]
    s = np.where(mask, s, -np.inf)
    m = np.max(s, axis=-1) if t1 > t0 else np.full(s.shape[:-1], -np.inf)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe[..., None])
    l = np.sum(e, axis=-1)
    acc = np.matmul(e, np.asarray(c_kv[t0:t1], dtype=np.float64))
    return m, l, acc


def merge_partials(parts):
    """Merge (m_k, l_k, acc_k) partials of disjoint key ranges:
    M = max_k m_k, o = sum_k e^{m_k-M} acc_k / sum_k e^{m_k-M} l_k,
    lse = M + log sum_k e^{m_k-M} l_k. Returns (o_lat, lse)."""
    ms = np.stack([p[0] for p in parts])
    M = np.max(ms, axis=0)
    M_safe = np.where(np.isfinite(M), M, 0.0)
    w = np.exp(ms - M_safe[None])
    l = np.sum(w * np.stack([p[1] for p in parts]), axis=0)
    acc = np.sum(w[..., None] * np.stack([p[2] for p in parts]), axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.where(l[..., None] > 0, acc / np.where(l > 0, l, 1.0)[..., None], 0.0)
        lse = np.where(l > 0, M_safe + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse


# --------------------------------------------------------------------------
# cache accounting ([MLA80] §1 table; [AUDIT] §2.1, §4; [TRACE] §3.2)


def mla_cache_elems_per_token(d_c: int = D_C, d_rope: int = D_ROPE) -> int:
    """Latent cache elements per token per layer: d_c + d_r ([MLA80] §1)."""
    return d_c + d_rope


def expanded_cache_elems_per_token(n_heads: int, d_nope: int = D_NOPE, d_rope: int = D_ROPE,
                                   d_v: int = D_V) -> int:
    """Naive expanded cache: key n_h*(d_nope+d_rope) + value n_h*d_v ([AUDIT] §2.1)."""
    return n_heads * (d_nope + d_rope) + n_heads * d_v


def mha_bytes_per_token(n_h: int, d_h: int, elt: int = 2) -> int:
    """MHA cache bytes per token per layer: 2 * n_h * d_h * elt ([MLA80] §1)."""
    return 2 * n_h * d_h * elt


def gqa_bytes_per_token(n_kv: int, d_h: int, elt: int = 2) -> int:
    """GQA cache bytes per token per layer: 2 * n_kv * d_h * elt ([MLA80] §1)."""
    return 2 * n_kv * d_h * elt


def mla_bytes_per_token(d_c: int = D_C, d_rope: int = D_ROPE, elt: int = 2) -> int:
    """MLA cache bytes per token per layer: (d_c + d_r) * elt ([MLA80] §1)."""
    return mla_cache_elems_per_token(d_c, d_rope) * elt


def cache_bytes(L: int, per_token_bytes: int) -> int:
    """Active cache bytes of L tokens."""
    return L * per_token_bytes


def paged_allocated_bytes(L: int, per_token_bytes: int, block: int = BLOCK) -> int:
    """Bytes held by a paged cache of L tokens: whole blocks of ``block`` rows."""
    return -(-L // block) * block * per_token_bytes
