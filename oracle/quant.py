"""Oracle: latent-cache quantisers and page layouts.  Test infrastructure only.

[Report] §3.2 compares quantisation schemes for the 512-wide latent and the
64-wide RoPE key; §4.1 keeps two of them: INT8 with one scale per 32-element
block, and asymmetric INT4 with a scale and a zero point per 32-element block.
The RoPE key is kept as INT8 in 8-element blocks.  The page does not fix the
arithmetic; the readings taken here (each one quantises a single appended token
by itself, so append can be done token by token) are:

  INT8 (symmetric, group of g consecutive channels of one token):
      amax  = max |x|                       (float32; exact from bf16)
      scale = amax / 127                    (IEEE float32 division, RNE)
      code  = clamp(rint(x / scale), -127, 127), rint = round half to even
      amax == 0  ->  scale = 0, codes 0;    dequant: code * scale (float32)
  INT4 (asymmetric, group of 32):
      mn, mx = min x, max x
      scale = (mx - mn) / 15                (float32)
      zero  = mn
      q     = clamp(rint((x - mn) / scale), 0, 15);  scale == 0 -> q = 0
      dequant: q * scale + zero (float32, two roundings)
      byte j of a token holds element 2j in bits 0-3 and 2j+1 in bits 4-7.
  INT8 per token (a variant the report does not measure): the INT8 reading
  with one group of all 512 latent channels; the RoPE key as for INT8.
  INT4 symmetric (a variant the report does not measure; the analogue of the
  INT8 reading with 4 bits), group of 32:
      amax = max |x|, scale = amax / 7      (float32)
      q = clamp(rint(x / scale), -7, 7);  amax == 0 -> scale 0, q 0
      stored as the nibble q + 8 (1..15), same byte order as INT4
      dequant: (nibble - 8) * scale (float32, one rounding)
  INT4 symmetric with an INT4 RoPE key (a variant the report does not
  measure): the latent as INT4 symmetric; the RoPE key by the same rule in
  groups of 8 (scale = max|x| / 7, nibble q + 8, same byte order).
  INT8 per channel over 32-token blocks (the report's "per-channel INT8 (32
  blocks)", which §4.1 keeps as its production setting): the 32 consecutive
  tokens of a block (positions 32j .. 32j + 31 of a sequence) share, for each
  latent channel c, one scale over the block:
      amax_c = max_t |x[t][c]|, scale_c = amax_c / 127 (float32),
      code = clamp(rint(x / scale_c), -127, 127); amax_c == 0 -> scale 0, codes 0
  (the INT8 reading applied down a channel instead of along a token).  A block
  is quantised when its 32nd token is appended; until then its tokens' latent
  rows are kept in bf16 (the "open" block, at most one per sequence).  The
  RoPE key is INT8 per token in 8-element groups, as for the other INT8 formats.
  FP8 per token (e4m3; a cache format the pages name but do not specify):
      amax = max |x| over the token's 512 latent channels (8 for each RoPE-key
      group), scale = amax / 448 (float32; 448 is the largest e4m3 value)
      code = e4m3(x / scale): round to nearest, ties to even, onto the e4m3
      grid (bias 7, 3 mantissa bits, subnormal step 2^-9, no infinities),
      saturating at +-448; the sign bit is the sign bit of x / scale
      amax == 0 -> scale 0, codes 0;  dequant: value(code) * scale (float32)

Every step is evaluated in numpy float32 with float32 constants, so the codes and
scales are defined bit for bit; the GPU's quantise-on-append must reproduce them
exactly.

Page layouts (64 tokens a page, bytes):
  bf16 : [64][576] bf16 (latent 0..511 then RoPE key 512..575)        73,728
  int8 : [64][576] int8 codes | [64][16] f32 latent scales
         | [64][8] f32 RoPE-key scales                                 43,008
  int4 : [64][256] packed latent nibbles | [64][64] int8 RoPE-key codes
         | [64][16] f32 scales | [64][16] f32 zeros
         | [64][8] f32 RoPE-key scales                                 30,720
  int4s: as int4 without the zeros                                    26,624
  int8t: [64][576] int8 codes | [64] f32 latent scales
         | [64][8] f32 RoPE-key scales                                 39,168
  fp8t : as int8t with e4m3 codes                                     39,168
  int4k4: [64][256] latent nibbles | [64][32] RoPE-key nibbles
         | [64][16] f32 scales | [64][8] f32 RoPE-key scales           24,576
  int8c: [64][512] int8 latent codes | [64][64] int8 RoPE-key codes
         | [2][512] f32 channel scales of blocks 0 and 1
         | [64][8] f32 RoPE-key scales | [32][512 B] overflow          59,392
         An open block b keeps its bf16 latent rows in place of its codes:
         channels 0..255 of row r in code row 32 b + r (512 B), channels
         256..511 in overflow row r.  Bytes the decode reads per closed token:
         512 + 64 + 64 (block scales, 2,048 B per 32 tokens) + 32 = 672.

Parity pins (tests/test_oracle_quant.py): the absmax element maps to +-127; an
INT4 group's min maps to 0 and its max to 15; the reconstruction error of every
unclamped element is at most half a step; zero groups round-trip exactly;
the rounding rule is checked on hand-made ties; page bytes round-trip through
unpack_page; a symmetric INT4 group's absmax element maps to nibble 8 +- 7;
the e4m3 encoder agrees with torch's float8_e4m3fn conversion, returns every
one of the 254 finite codes from its own value, rounds hand-made midpoints to
the even code, and maps a group's absmax element to +-448.  The
page's own error figures need the real latents and are not reproduced ("parity
unpinned" for those numbers).
"""
from __future__ import annotations

import numpy as np

BLOCK = 64
D_C = 512
D_R = 64
G_C = 32      # latent channels per group
G_R = 8       # RoPE-key channels per group

CACHE_BF16, CACHE_INT8, CACHE_INT4, CACHE_INT4_SYM, CACHE_INT8_TOK, CACHE_FP8_TOK, CACHE_INT4_SYM_K4, CACHE_INT8_CHAN = range(8)
T_BLK = 32    # tokens per channel-scale block of the int8c format
_F448 = np.float32(448.0)
_F127 = np.float32(127.0)
_F15 = np.float32(15.0)
_F7 = np.float32(7.0)


def _bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def quant_int8_sym(x_bits: np.ndarray, group: int):
    """Symmetric INT8 per group of `group` consecutive channels of each row.

    x_bits [..., C] bf16 bits -> codes int8 [..., C], scales float32 [..., C/group]
    """
    x = _bf16_to_f32(x_bits)
    shp = x.shape
    xg = x.reshape(shp[:-1] + (shp[-1] // group, group))
    amax = np.max(np.abs(xg), axis=-1)                         # float32
    scale = (amax / _F127).astype(np.float32)
    safe = np.where(scale == 0, np.float32(1.0), scale).astype(np.float32)
    q = np.rint((xg / safe[..., None]).astype(np.float32))
    q = np.clip(q, -127, 127)
    q = np.where(scale[..., None] == 0, 0, q)
    return q.astype(np.int8).reshape(shp), scale


def dequant_int8(codes: np.ndarray, scales: np.ndarray, group: int) -> np.ndarray:
    shp = codes.shape
    cg = codes.astype(np.float32).reshape(shp[:-1] + (shp[-1] // group, group))
    return (cg * scales[..., None].astype(np.float32)).astype(np.float32).reshape(shp)


def fp8_e4m3_encode(y: np.ndarray) -> np.ndarray:
    """float32 -> e4m3 code bytes: nearest grid value (ties to even), saturating at 448."""
    y = np.asarray(y, np.float32)
    a = np.abs(y)
    _, k = np.frexp(a)                                       # a = f 2^k, 0.5 <= f < 1
    e = np.maximum(k.astype(np.int32) - 1, -6)               # 2^e <= a < 2^(e+1) for normals
    sub = a < np.float32(2.0 ** -6)
    q_sub = np.rint(a * np.float32(512.0))                   # multiples of 2^-9 (exact scaling)
    q_nrm = np.rint(np.ldexp(a, 3 - e).astype(np.float32))   # 8..16: 1.mmm in units of 1/8
    code = np.where(sub, q_sub, (e + 7) * 8 + (q_nrm - 8))   # q = 16 carries into the exponent
    code = np.minimum(code, 126).astype(np.uint8)
    return np.where(np.signbit(y), code | np.uint8(0x80), code).astype(np.uint8)


def fp8_e4m3_decode(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, np.uint8).astype(np.int32)
    E, M = (c >> 3) & 15, c & 7
    v = np.where(E == 0, M * np.float32(2.0 ** -9),
                 np.ldexp(np.float32(1.0) + M.astype(np.float32) / np.float32(8.0), E - 7)).astype(np.float32)
    return np.where(c >> 7 == 1, -v, v).astype(np.float32)


def quant_fp8(x_bits: np.ndarray, group: int):
    """e4m3 codes per group of `group` channels with scale = amax / 448."""
    x = _bf16_to_f32(x_bits)
    shp = x.shape
    xg = x.reshape(shp[:-1] + (shp[-1] // group, group))
    amax = np.max(np.abs(xg), axis=-1)
    scale = (amax / _F448).astype(np.float32)
    safe = np.where(scale == 0, np.float32(1.0), scale).astype(np.float32)
    codes = fp8_e4m3_encode((xg / safe[..., None]).astype(np.float32))
    codes = np.where(scale[..., None] == 0, np.uint8(0), codes).astype(np.uint8)
    return codes.reshape(shp), scale


def dequant_fp8(codes: np.ndarray, scales: np.ndarray, group: int) -> np.ndarray:
    shp = codes.shape
    v = fp8_e4m3_decode(codes).reshape(shp[:-1] + (shp[-1] // group, group))
    return (v * scales[..., None].astype(np.float32)).astype(np.float32).reshape(shp)


def quant_int4_asym(x_bits: np.ndarray, group: int = G_C):
    """Asymmetric INT4 per group: returns q uint8 [..., C] (0..15), scale, zero float32."""
    x = _bf16_to_f32(x_bits)
    shp = x.shape
    xg = x.reshape(shp[:-1] + (shp[-1] // group, group))
    mn = np.min(xg, axis=-1)
    mx = np.max(xg, axis=-1)
    scale = (mx - mn).astype(np.float32) / _F15
    scale = scale.astype(np.float32)
    safe = np.where(scale == 0, np.float32(1.0), scale).astype(np.float32)
    d = (xg - mn[..., None]).astype(np.float32)
    q = np.rint((d / safe[..., None]).astype(np.float32))
    q = np.clip(q, 0, 15)
    q = np.where(scale[..., None] == 0, 0, q)
    return q.astype(np.uint8).reshape(shp), scale, mn.astype(np.float32)


def dequant_int4(q: np.ndarray, scale: np.ndarray, zero: np.ndarray, group: int = G_C) -> np.ndarray:
    shp = q.shape
    qg = q.astype(np.float32).reshape(shp[:-1] + (shp[-1] // group, group))
    prod = (qg * scale[..., None].astype(np.float32)).astype(np.float32)
    return (prod + zero[..., None].astype(np.float32)).astype(np.float32).reshape(shp)


def quant_int4_sym(x_bits: np.ndarray, group: int = G_C):
    """Symmetric INT4 per group: returns nibbles uint8 [..., C] (q + 8, 1..15) and scale float32."""
    x = _bf16_to_f32(x_bits)
    shp = x.shape
    xg = x.reshape(shp[:-1] + (shp[-1] // group, group))
    amax = np.max(np.abs(xg), axis=-1)
    scale = (amax / _F7).astype(np.float32)
    safe = np.where(scale == 0, np.float32(1.0), scale).astype(np.float32)
    q = np.rint((xg / safe[..., None]).astype(np.float32))
    q = np.clip(q, -7, 7)
    q = np.where(scale[..., None] == 0, 0, q)
    return (q + 8).astype(np.uint8).reshape(shp), scale


def dequant_int4_sym(nib: np.ndarray, scale: np.ndarray, group: int = G_C) -> np.ndarray:
    shp = nib.shape
    qg = (nib.astype(np.float32) - np.float32(8.0)).reshape(shp[:-1] + (shp[-1] // group, group))
    return (qg * scale[..., None].astype(np.float32)).astype(np.float32).reshape(shp)


def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """[..., 2n] values 0..15 -> [..., n] bytes: element 2j low nibble, 2j+1 high."""
    q = q.astype(np.uint8)
    return (q[..., 0::2] | (q[..., 1::2] << np.uint8(4))).astype(np.uint8)


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = b & np.uint8(0x0F)
    out[..., 1::2] = b >> np.uint8(4)
    return out


def token_bytes(dtype: int) -> int:
    """Cache bytes per token including scales and zero points."""
    return {CACHE_BF16: 576 * 2,
            CACHE_INT8: 576 + (D_C // G_C) * 4 + (D_R // G_R) * 4,
            CACHE_INT4: D_C // 2 + D_R + (D_C // G_C) * 8 + (D_R // G_R) * 4,
            CACHE_INT4_SYM: D_C // 2 + D_R + (D_C // G_C) * 4 + (D_R // G_R) * 4,
            CACHE_INT8_TOK: 576 + 4 + (D_R // G_R) * 4,
            CACHE_FP8_TOK: 576 + 4 + (D_R // G_R) * 4,
            CACHE_INT4_SYM_K4: D_C // 2 + D_R // 2 + (D_C // G_C) * 4 + (D_R // G_R) * 4,
            CACHE_INT8_CHAN: D_C + D_R + D_C * 4 // T_BLK + (D_R // G_R) * 4}[dtype]


def page_bytes(dtype: int) -> int:
    if dtype == CACHE_INT8_CHAN:
        return BLOCK * (D_C + D_R + (D_R // G_R) * 4) + 2 * D_C * 4 + T_BLK * D_C
    return BLOCK * token_bytes(dtype)


def quant_int8_channel_block(x_bits: np.ndarray):
    """One closed block: x_bits [32, C] bf16 bits -> codes int8 [32, C] and one
    float32 scale per channel [C], by the INT8 rule applied down each channel."""
    assert x_bits.shape[0] == T_BLK
    q, s = quant_int8_sym(np.ascontiguousarray(x_bits.T), T_BLK)
    return np.ascontiguousarray(q.T), s[:, 0]


def _encode_int8_chan(c_bits: np.ndarray, r_bits: np.ndarray) -> dict:
    """Rows 0..n-1 of a sequence from a block boundary on: full 32-row blocks are
    closed (codes + channel scales), a trailing partial block stays open (bf16)."""
    n = c_bits.shape[0]
    n_closed = (n // T_BLK) * T_BLK
    codes = np.zeros((n, D_C), np.int8)
    scales = np.zeros((n_closed // T_BLK, D_C), np.float32)
    for j in range(n_closed // T_BLK):
        codes[j * T_BLK:(j + 1) * T_BLK], scales[j] = quant_int8_channel_block(c_bits[j * T_BLK:(j + 1) * T_BLK])
    rc, rs = quant_int8_sym(r_bits, G_R)
    return {"codes": codes, "blk_scale": scales, "r_codes": rc, "r_scale": rs,
            "open": np.asarray(c_bits[n_closed:], np.uint16).copy(), "n_closed": n_closed}


def encode_tokens(dtype: int, c_bits: np.ndarray, r_bits: np.ndarray) -> dict:
    """Quantise (or copy) n token rows into their per-field arrays."""
    if dtype == CACHE_BF16:
        return {"rows": np.concatenate([c_bits, r_bits], axis=-1).astype(np.uint16)}
    if dtype == CACHE_INT8_CHAN:
        return _encode_int8_chan(c_bits, r_bits)
    if dtype == CACHE_INT4_SYM_K4:
        q, s = quant_int4_sym(c_bits, G_C)
        rq, rs = quant_int4_sym(r_bits, G_R)
        return {"nib": pack_nibbles(q), "r_nib": pack_nibbles(rq), "c_scale": s, "r_scale": rs}
    if dtype == CACHE_FP8_TOK:
        cc, cs = quant_fp8(c_bits, D_C)
        rc, rs = quant_fp8(r_bits, G_R)
        return {"codes": np.concatenate([cc, rc], axis=-1), "c_scale": cs, "r_scale": rs}
    rc, rs = quant_int8_sym(r_bits, G_R)
    if dtype in (CACHE_INT8, CACHE_INT8_TOK):
        cc, cs = quant_int8_sym(c_bits, G_C if dtype == CACHE_INT8 else D_C)
        return {"codes": np.concatenate([cc, rc], axis=-1), "c_scale": cs, "r_scale": rs}
    if dtype == CACHE_INT4_SYM:
        q, s = quant_int4_sym(c_bits, G_C)
        return {"nib": pack_nibbles(q), "r_codes": rc, "c_scale": s, "r_scale": rs}
    q, s, z = quant_int4_asym(c_bits, G_C)
    return {"nib": pack_nibbles(q), "r_codes": rc, "c_scale": s, "c_zero": z, "r_scale": rs}


def pack_page(dtype: int, fields: dict) -> np.ndarray:
    """Lay out the fields of up to 64 tokens as one page (uint8 [page_bytes]).

    Slots beyond the tokens given are zero.
    """
    out = np.zeros(page_bytes(dtype), np.uint8)

    def put(off, arr, width):
        a = np.ascontiguousarray(arr).view(np.uint8).reshape(-1, width)
        out[off: off + a.size] = a.reshape(-1)
        return off + BLOCK * width

    if dtype == CACHE_BF16:
        put(0, fields["rows"], 1152)
    elif dtype == CACHE_INT8_CHAN:
        nc = fields["n_closed"]
        off = put(0, fields["codes"][:nc], 512)
        op = fields["open"]
        if len(op):                                    # open block b = nc // 32 of this page
            row0 = nc
            halves = np.ascontiguousarray(op[:, :D_C // 2]).view(np.uint8).reshape(-1)
            out[row0 * 512: row0 * 512 + halves.size] = halves
            tail = np.ascontiguousarray(op[:, D_C // 2:]).view(np.uint8).reshape(-1)
            base = BLOCK * (D_C + D_R + (D_R // G_R) * 4) + 2 * D_C * 4
            out[base: base + tail.size] = tail
        off = put(off, fields["r_codes"], 64)
        sc = np.ascontiguousarray(fields["blk_scale"]).view(np.uint8).reshape(-1)
        out[off: off + sc.size] = sc
        off += 2 * D_C * 4
        put(off, fields["r_scale"], 32)
    elif dtype in (CACHE_INT8, CACHE_INT8_TOK, CACHE_FP8_TOK):
        off = put(0, fields["codes"], 576)
        off = put(off, fields["c_scale"], 64 if dtype == CACHE_INT8 else 4)
        put(off, fields["r_scale"], 32)
    elif dtype == CACHE_INT4_SYM_K4:
        off = put(0, fields["nib"], 256)
        off = put(off, fields["r_nib"], 32)
        off = put(off, fields["c_scale"], 64)
        put(off, fields["r_scale"], 32)
    else:
        off = put(0, fields["nib"], 256)
        off = put(off, fields["r_codes"], 64)
        off = put(off, fields["c_scale"], 64)
        if dtype == CACHE_INT4:
            off = put(off, fields["c_zero"], 64)
        put(off, fields["r_scale"], 32)
    return out


def unpack_page(dtype: int, page: np.ndarray) -> dict:
    """Inverse of pack_page for all 64 slots."""
    page = np.asarray(page, np.uint8)

    def get(off, width, dt, cols):
        raw = page[off: off + BLOCK * width].copy()
        return raw.view(dt).reshape(BLOCK, cols), off + BLOCK * width

    if dtype == CACHE_BF16:
        rows, _ = get(0, 1152, np.uint16, 576)
        return {"rows": rows}
    if dtype == CACHE_INT8_CHAN:
        codes, off = get(0, 512, np.int8, 512)
        rc, off = get(off, 64, np.int8, 64)
        sc = page[off: off + 2 * D_C * 4].copy().view(np.float32).reshape(2, D_C)
        off += 2 * D_C * 4
        rs, off = get(off, 32, np.float32, 8)
        ov = page[off: off + T_BLK * D_C].copy().view(np.uint16).reshape(T_BLK, D_C // 2)
        return {"codes": codes, "r_codes": rc, "blk_scale": sc, "r_scale": rs, "overflow": ov}
    if dtype in (CACHE_INT8, CACHE_INT8_TOK, CACHE_FP8_TOK):
        codes, off = get(0, 576, np.uint8 if dtype == CACHE_FP8_TOK else np.int8, 576)
        cs, off = get(off, 64, np.float32, 16) if dtype == CACHE_INT8 else get(off, 4, np.float32, 1)
        rs, _ = get(off, 32, np.float32, 8)
        return {"codes": codes, "c_scale": cs, "r_scale": rs}
    nib, off = get(0, 256, np.uint8, 256)
    if dtype == CACHE_INT4_SYM_K4:
        rn, off = get(off, 32, np.uint8, 32)
        cs, off = get(off, 64, np.float32, 16)
        rs, _ = get(off, 32, np.float32, 8)
        return {"nib": nib, "r_nib": rn, "c_scale": cs, "r_scale": rs}
    rc, off = get(off, 64, np.int8, 64)
    cs, off = get(off, 64, np.float32, 16)
    if dtype == CACHE_INT4_SYM:
        rs, _ = get(off, 32, np.float32, 8)
        return {"nib": nib, "r_codes": rc, "c_scale": cs, "r_scale": rs}
    cz, off = get(off, 64, np.float32, 16)
    rs, _ = get(off, 32, np.float32, 8)
    return {"nib": nib, "r_codes": rc, "c_scale": cs, "c_zero": cz, "r_scale": rs}


def dequant_fields(dtype: int, f: dict):
    """Fields of n tokens -> (c [n,512], r [n,64]) float32 values the decode reads."""
    if dtype == CACHE_BF16:
        rows = _bf16_to_f32(f["rows"])
        return rows[..., :D_C], rows[..., D_C:]
    if dtype == CACHE_INT8_CHAN:
        nc = f["n_closed"]
        c = np.zeros((nc + len(f["open"]), D_C), np.float32)
        for j in range(nc // T_BLK):
            c[j * T_BLK:(j + 1) * T_BLK] = (f["codes"][j * T_BLK:(j + 1) * T_BLK].astype(np.float32)
                                            * f["blk_scale"][j][None, :]).astype(np.float32)
        c[nc:] = _bf16_to_f32(f["open"])
        return c, dequant_int8(f["r_codes"], f["r_scale"], G_R)
    if dtype == CACHE_FP8_TOK:
        return dequant_fp8(f["codes"][..., :D_C], f["c_scale"], D_C), dequant_fp8(f["codes"][..., D_C:], f["r_scale"], G_R)
    if dtype in (CACHE_INT8, CACHE_INT8_TOK):
        c = dequant_int8(f["codes"][..., :D_C], f["c_scale"], G_C if dtype == CACHE_INT8 else D_C)
        r = dequant_int8(f["codes"][..., D_C:], f["r_scale"], G_R)
        return c, r
    if dtype == CACHE_INT4_SYM_K4:
        return (dequant_int4_sym(unpack_nibbles(f["nib"]), f["c_scale"], G_C),
                dequant_int4_sym(unpack_nibbles(f["r_nib"]), f["r_scale"], G_R))
    if dtype == CACHE_INT4_SYM:
        c = dequant_int4_sym(unpack_nibbles(f["nib"]), f["c_scale"], G_C)
    else:
        c = dequant_int4(unpack_nibbles(f["nib"]), f["c_scale"], f["c_zero"], G_C)
    r = dequant_int8(f["r_codes"], f["r_scale"], G_R)
    return c, r


def pack_pool(dtype: int, num_pages: int, seqs) -> np.ndarray:
    """Build a whole pool from (c_bits [L,512], r_bits [L,64], block_table_row) triples."""
    pool = np.zeros((num_pages, page_bytes(dtype)), np.uint8)
    for c_bits, r_bits, bt_row in seqs:
        L = c_bits.shape[0]
        for p0 in range(0, L, BLOCK):
            n = min(BLOCK, L - p0)
            f = encode_tokens(dtype, c_bits[p0:p0 + n], r_bits[p0:p0 + n])
            pool[int(bt_row[p0 // BLOCK])] = pack_page(dtype, f)
    return pool


def page_fields_int8_chan(page: np.ndarray, n: int) -> dict:
    """The fields an int8c page holds for its first n tokens (the layout read back
    the way encode_tokens returns it: closed codes and scales, open rows)."""
    u = unpack_page(CACHE_INT8_CHAN, page)
    nc = (n // T_BLK) * T_BLK
    codes = np.zeros((n, D_C), np.int8)
    codes[:nc] = u["codes"][:nc]
    op = np.zeros((n - nc, D_C), np.uint16)
    if n > nc:
        op[:, :D_C // 2] = u["codes"][nc:n].view(np.uint16)
        op[:, D_C // 2:] = u["overflow"][: n - nc]
    return {"codes": codes, "blk_scale": u["blk_scale"][: nc // T_BLK].copy(), "r_codes": u["r_codes"][:n].copy(),
            "r_scale": u["r_scale"][:n].copy(), "open": op, "n_closed": nc}


def dequant_pool_seq(dtype: int, pool: np.ndarray, bt_row: np.ndarray, L: int):
    """Read one sequence back from a packed pool: (c [L,512], r [L,64]) float64."""
    cs, rs = [], []
    for p0 in range(0, L, BLOCK):
        n = min(BLOCK, L - p0)
        f = unpack_page(dtype, pool[int(bt_row[p0 // BLOCK])])
        c, r = dequant_fields(dtype, f)
        cs.append(c[:n])
        rs.append(r[:n])
    return (np.concatenate(cs).astype(np.float64), np.concatenate(rs).astype(np.float64))
