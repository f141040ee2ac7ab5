"""Byte layout of one packed (16-token block, kv-head) record.

Test infrastructure only (see ``oracle/__init__``).  Written from the layout
definition (the same text that the C header documents); it shares no code with
the kernels.

The pages fix only the block size: vLLM paged KV blocks of 16 tokens ([ST],
first body paragraph after the summary).  Everything else below is this
project's format.  Pools are laid out [num_blocks][num_kv_heads][record].

Nibbles: a byte holds two 4-bit codes, the even channel (or the first of the
pair) in the low nibble.  fp16 values are little-endian.  D = head_dim,
P = D/2 channel pairs (pair p = channels 2p, 2p+1), Q = D/8, G = D/32 groups,
token row t in [0, 16), t = 4r + tt.

TQ4/4 record (D = 64 or 128), sections in this order:
  Kc  16*P bytes  key codes:     pair p of token t at  ((p // Q) * 16 + t) * Q + p % Q
  Vc  16*P bytes  value codes:   pair p = 16*gp + j of token t at ((r*16 + j)*G + gp)*4 + tt
  Vm  16*G*4 B    value scale/min:
                   sc(t, gp) at 2*((r*G + gp)*8 + tt),  mn(t, gp) at 2*((r*G + gp)*8 + 4 + tt)
  Ks  16*2 bytes  key scales:    fp16 s_t at byte 2t
  Payload 16 * (D/2 + D/2 + G*4 + 2) bytes: 2336 (D=128), 1184 (D=64).  At
  D = 128 the record is padded with unused bytes to whole 128-byte lines: 2432.

TQ4/2 record (D = 64 or 128; 2-bit values), sections in this order:
  Kc  16*P bytes  as TQ4/4
  Vc2 16*P/2 B    2-bit value codes: channel 2p + par, p = 16*gp + j, of token
                  t in byte ((r*16 + j)*(G/2) + gp//2)*4 + tt at bit 4*(gp%2) + 2*par
  Vm  16*G*4 B    as TQ4/4
  Ks  16*2 bytes  as TQ4/4
  Payload 16 * (D/2 + D/4 + G*4 + 2) bytes: 1824 (D=128), 928 (D=64); padded
  to 1920 at D = 128.

MX-FP4 record (D = 128 only), sections in this order:
  Kc4 16*P bytes  e2m1 key codes (rotated keys), same placement as Kc
  Vc4 16*P bytes  e2m1 value codes, same placement as Vc
  Ks4 16*G bytes  UE8M0 key exponents: group gp of token t at gp*16 + t
  Vs4 16*G bytes  UE8M0 value exponents: group gp of token t at (r*G + gp)*4 + tt
  Record bytes: 2176 (D=128) = 16 * (D/2 + D/2 + G + G), whole 128-byte lines.

The large sections start on 128-byte boundaries of a record, and at D = 128
the records themselves do (an implementation choice of this format: writes of
whole lines).

Pinned by tests/test_oracle_layout.py: hand-written byte examples, every
section offset map is a bijection onto its section, nibble pack/unpack over all
256 byte values.
"""
import numpy as np

BLOCK = 16


def _lines(n):
    """n rounded up to whole 128-byte lines."""
    return (n + 127) // 128 * 128


def tq4_record_bytes(d):
    return tq4_sections(d)["bytes"]


def tq4v2_record_bytes(d):
    return tq4v2_sections(d)["bytes"]


def mxfp4_record_bytes(d):
    return mxfp4_sections(d)["bytes"]


def _check_dim(d):
    if d not in (64, 128):
        raise ValueError("head_dim must be 64 or 128")


# --- section offsets (relative to the section start) -------------------------

def kc_offset(t, p, d):
    q = d // 8
    t = np.asarray(t)
    p = np.asarray(p)
    return ((p // q) * BLOCK + t) * q + p % q


def vc_offset(t, p, d):
    g = d // 32
    t = np.asarray(t)
    p = np.asarray(p)
    r, tt = t // 4, t % 4
    gp, j = p // 16, p % 16
    return ((r * 16 + j) * g + gp) * 4 + tt


def vc2_position(t, c, d):
    """(byte offset in the Vc2 section, bit shift) of the 2-bit code of
    channel c of token t."""
    g = d // 32
    t = np.asarray(t)
    c = np.asarray(c)
    r, tt = t // 4, t % 4
    p, par = c // 2, c % 2
    gp, j = p // 16, p % 16
    return ((r * 16 + j) * (g // 2) + gp // 2) * 4 + tt, 4 * (gp % 2) + 2 * par


def vm_offsets(t, gp, d):
    """(scale byte offset, min byte offset) of group gp of token t."""
    g = d // 32
    t = np.asarray(t)
    gp = np.asarray(gp)
    r, tt = t // 4, t % 4
    base = (r * g + gp) * 8
    return 2 * (base + tt), 2 * (base + 4 + tt)


def ks4_offset(t, gp):
    return np.asarray(gp) * BLOCK + np.asarray(t)


def vs4_offset(t, gp, d):
    g = d // 32
    t = np.asarray(t)
    return ((t // 4) * g + np.asarray(gp)) * 4 + t % 4


def tq4_sections(d):
    """Start byte of each section of a TQ4 record; "end": end of the payload,
    "bytes": the record size (D = 128: whole 128-byte lines)."""
    _check_dim(d)
    p16 = BLOCK * (d // 2)
    kc = 0
    vc = kc + p16
    vm = vc + p16
    ks = vm + BLOCK * (d // 32) * 4
    end = ks + 2 * BLOCK
    return {"kc": kc, "vc": vc, "vm": vm, "ks": ks, "end": end, "bytes": _lines(end) if d == 128 else end}


def tq4v2_sections(d):
    """Start byte of each section of a TQ4/2 record (keys as in TQ4/4)."""
    _check_dim(d)
    p16 = BLOCK * (d // 2)
    kc = 0
    vc = kc + p16
    vm = vc + p16 // 2
    ks = vm + BLOCK * (d // 32) * 4
    end = ks + 2 * BLOCK
    return {"kc": kc, "vc": vc, "vm": vm, "ks": ks, "end": end, "bytes": _lines(end) if d == 128 else end}


def mxfp4_sections(d):
    if d != 128:
        raise ValueError("the MX-FP4 record is defined for head_dim 128")
    p16 = BLOCK * (d // 2)
    g16 = BLOCK * (d // 32)
    kc = 0
    vc = kc + p16
    ks = vc + p16
    vs = ks + g16
    end = vs + g16
    return {"kc": kc, "vc": vc, "ks": ks, "vs": vs, "end": end, "bytes": end}


# --- nibbles -----------------------------------------------------------------

def pack_nibbles(codes):
    """[..., 2n] 4-bit codes -> [..., n] bytes, even element in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    if np.any(c > 15):
        raise ValueError("codes must be 4-bit")
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(b):
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


# --- whole-row writers and readers ----------------------------------------------
# Writers scatter into a flat byte buffer ``buf``: row i goes into the record
# that starts at byte ``base[i]``, token row ``t[i]``.  Distinct (record, row)
# pairs never share a byte, so rows of one block can be written together.

def _put_f16(buf, pos, val):
    bits = np.asarray(val, dtype=np.float16).view(np.uint16)
    buf[pos] = (bits & 0xFF).astype(np.uint8)
    buf[pos + 1] = (bits >> 8).astype(np.uint8)


def tq4_write_rows(buf, base, t, d, kcode, kscale, vcode, vscale, vmin):
    sec = tq4_sections(d)
    base = np.asarray(base, dtype=np.int64).reshape(-1, 1)
    n = base.shape[0]
    t = np.asarray(t).reshape(n, 1)
    p = np.arange(d // 2)[None, :]
    buf[base + sec["kc"] + kc_offset(t, p, d)] = pack_nibbles(kcode).reshape(n, d // 2)
    buf[base + sec["vc"] + vc_offset(t, p, d)] = pack_nibbles(vcode).reshape(n, d // 2)
    _put_f16(buf, (base + sec["ks"] + 2 * t).ravel(), np.asarray(kscale).reshape(n))
    gp = np.arange(d // 32)[None, :]
    so, mo = vm_offsets(t, gp, d)
    _put_f16(buf, base + sec["vm"] + so, np.asarray(vscale).reshape(n, d // 32))
    _put_f16(buf, base + sec["vm"] + mo, np.asarray(vmin).reshape(n, d // 32))


def tq4_read_block(rec, d):
    """Decode the sections of records ``rec`` [n, bytes] into per-token arrays
    (kcode [n,16,D], kscale [n,16], vcode [n,16,D], vscale/vmin [n,16,G])."""
    sec = tq4_sections(d)
    rec = np.asarray(rec, dtype=np.uint8)
    n = rec.shape[0]
    t = np.arange(BLOCK)[:, None]
    p = np.arange(d // 2)[None, :]
    kb = rec[:, sec["kc"] + kc_offset(t, p, d)]
    vb = rec[:, sec["vc"] + vc_offset(t, p, d)]
    ksb = rec[:, sec["ks"]:sec["ks"] + 2 * BLOCK].copy().view(np.float16).reshape(n, BLOCK)
    g = d // 32
    so, mo = vm_offsets(np.arange(BLOCK)[:, None], np.arange(g)[None, :], d)

    def f16_at(off):
        lo = rec[:, sec["vm"] + off].astype(np.uint16)
        hi = rec[:, sec["vm"] + off + 1].astype(np.uint16)
        return (lo | (hi << 8)).view(np.float16)

    return {
        "kcode": unpack_nibbles(kb),
        "kscale": ksb,
        "vcode": unpack_nibbles(vb),
        "vscale": f16_at(so),
        "vmin": f16_at(mo),
    }


def tq4v2_write_rows(buf, base, t, d, kcode, kscale, vcode, vscale, vmin):
    """TQ4/2 rows: as tq4_write_rows, with 2-bit value codes [n, D]."""
    sec = tq4v2_sections(d)
    base = np.asarray(base, dtype=np.int64).reshape(-1, 1)
    n = base.shape[0]
    t = np.asarray(t).reshape(n, 1)
    p = np.arange(d // 2)[None, :]
    buf[base + sec["kc"] + kc_offset(t, p, d)] = pack_nibbles(kcode).reshape(n, d // 2)
    vcode = np.asarray(vcode, dtype=np.uint8).reshape(n, d)
    if np.any(vcode > 3):
        raise ValueError("codes must be 2-bit")
    pos, shift = vc2_position(t, np.arange(d)[None, :], d)
    pos = np.broadcast_to(base + sec["vc"] + pos, (n, d)).ravel()
    shift = np.broadcast_to(shift, (n, d)).ravel()
    # four codes of one token share a byte: assemble each byte, then store it
    where, inv = np.unique(pos, return_inverse=True)
    byte = np.zeros(where.shape, dtype=np.uint8)
    np.bitwise_or.at(byte, inv, (vcode.ravel() << shift).astype(np.uint8))
    buf[where] = byte
    _put_f16(buf, (base + sec["ks"] + 2 * t).ravel(), np.asarray(kscale).reshape(n))
    gp = np.arange(d // 32)[None, :]
    so, mo = vm_offsets(t, gp, d)
    _put_f16(buf, base + sec["vm"] + so, np.asarray(vscale).reshape(n, d // 32))
    _put_f16(buf, base + sec["vm"] + mo, np.asarray(vmin).reshape(n, d // 32))


def tq4v2_read_block(rec, d):
    """As tq4_read_block for TQ4/2 records (2-bit value codes)."""
    sec = tq4v2_sections(d)
    rec = np.asarray(rec, dtype=np.uint8)
    n = rec.shape[0]
    t = np.arange(BLOCK)[:, None]
    p = np.arange(d // 2)[None, :]
    kb = rec[:, sec["kc"] + kc_offset(t, p, d)]
    pos, shift = vc2_position(t, np.arange(d)[None, :], d)
    vcode = (rec[:, sec["vc"] + pos] >> shift) & 3
    ksb = rec[:, sec["ks"]:sec["ks"] + 2 * BLOCK].copy().view(np.float16).reshape(n, BLOCK)
    g = d // 32
    so, mo = vm_offsets(np.arange(BLOCK)[:, None], np.arange(g)[None, :], d)

    def f16_at(off):
        lo = rec[:, sec["vm"] + off].astype(np.uint16)
        hi = rec[:, sec["vm"] + off + 1].astype(np.uint16)
        return (lo | (hi << 8)).view(np.float16)

    return {"kcode": unpack_nibbles(kb), "kscale": ksb, "vcode": vcode.astype(np.uint8),
            "vscale": f16_at(so), "vmin": f16_at(mo)}


def mxfp4_write_rows(buf, base, t, d, kcode, kexp, vcode, vexp):
    """FP4 rows: e2m1 codes [n, D], UE8M0 exponents X [n, G] stored as X + 127."""
    sec = mxfp4_sections(d)
    base = np.asarray(base, dtype=np.int64).reshape(-1, 1)
    n = base.shape[0]
    t = np.asarray(t).reshape(n, 1)
    p = np.arange(d // 2)[None, :]
    gp = np.arange(d // 32)[None, :]
    buf[base + sec["kc"] + kc_offset(t, p, d)] = pack_nibbles(kcode).reshape(n, d // 2)
    buf[base + sec["vc"] + vc_offset(t, p, d)] = pack_nibbles(vcode).reshape(n, d // 2)
    buf[base + sec["ks"] + ks4_offset(t, gp)] = (np.asarray(kexp).reshape(n, -1) + 127).astype(np.uint8)
    buf[base + sec["vs"] + vs4_offset(t, gp, d)] = (np.asarray(vexp).reshape(n, -1) + 127).astype(np.uint8)


def mxfp4_read_block(rec, d):
    sec = mxfp4_sections(d)
    rec = np.asarray(rec, dtype=np.uint8)
    t = np.arange(BLOCK)[:, None]
    p = np.arange(d // 2)[None, :]
    gp = np.arange(d // 32)[None, :]
    return {
        "kcode": unpack_nibbles(rec[:, sec["kc"] + kc_offset(t, p, d)]),
        "kexp": rec[:, sec["ks"] + ks4_offset(t, gp)].astype(np.int64) - 127,
        "vcode": unpack_nibbles(rec[:, sec["vc"] + vc_offset(t, p, d)]),
        "vexp": rec[:, sec["vs"] + vs4_offset(t, gp, d)].astype(np.int64) - 127,
    }
