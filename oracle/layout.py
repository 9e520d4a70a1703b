"""Byte-exact device layout of the packed formats (oracle; test infrastructure).

The pages say only that engines repack checkpoints into an internal layout
(memra page, model/quantisation notes) and that 4-bit codes are packed as
nibbles along K. The layout below is this library's own, chosen so that one
16-byte load per lane of a 64-lane wave fetches one contiguous 1 KiB tile;
it is written out here independently of the library, from its specification.

Geometry
  Mp = M rounded up to 16, Kp = K rounded up to 128 (padding: code 0 and
  zero scale fields, i.e. weight 0). RT = Mp / 16 row tiles, KS = Kp / 128
  k-steps. Tile index tau = rt * KS + ks (row tiles outer, k-steps inner).
  In a tile, lane lam in [0, 64) has r = lam % 16 (row 16*rt + r) and
  s = lam // 16; for group j in [0, 4) and slot e in [0, 8) the lane holds
  column k = 128*ks + 32*j + 8*s + e.

int4   wq: tile = 1024 B; lane lam's 16 B at lam*16; dword j holds the 8
           codes of group j; code for slot e is nibble i (bits 4i..4i+3 of
           the little-endian dword) with i = e/2 for even e, 4 + (e-1)/2 for
           odd e.
       ws: tile = 256 B; row r's 16 B at r*16 hold the groups in the order
           j = 0, 2, 1, 3: dword at r*16 + 4*pos(j), pos(j) = 2*(j & 1) + (j >> 1),
           value fp16(d) | fp16(m) << 16.
int5   wq: plane A (RT*KS*1024 B: lane lam's 16 B at tau*1024 + lam*16 = dwords
           D0..D3), then plane B (RT*KS*256 B: lane lam's dword D4 at
           RT*KS*1024 + tau*256 + lam*4). The lane's 32 codes form 16 pairs
           P = 4*j + (e >> 1), half h = e & 1. For P < 15 the 5-bit code sits at
           bits 16*h + 5*c .. +4 of dword D(P // 3), c = P % 3. For P = 15, bit b
           of the code (b = 0..4) is bit 16*h + 15 of dword D(b).
       ws: as int4.
int8   wq: tile = 2048 B; byte (j >> 1)*1024 + lam*16 + (j & 1)*8 + e holds the
           code (two's complement).
       ws: tile = 128 B; fp16(d) at byte r*8 + 2*pos(j) (same group order).
nvfp4  wq: tile = 1024 B; byte lam*16 + 4*j + (e >> 1), low nibble for even e,
           high nibble for odd e (E2M1 codes).
       ws: tile = 128 B; byte r*8 + 4*h + j holds the E4M3 scale of the 16-block
           along K with index 8*ks + 2*j + h; after all tiles (offset
           RT*KS*128) the fp32 tensor scale, then 12 zero bytes.

MX formats: the operand layout of gfx950's block-scaled 16x16x128 MFMA, so
that each lane's load is its operand register as is (lane lam: row
16*rt + lam % 16, g = lam // 16):
mxfp8  wq: tile = 2048 B; byte h*1024 + lam*16 + i (h in {0, 1}, i < 16) holds
           the E4M3 code of column 128*ks + 64*h + 16*g + i.
mxfp4  wq: tile = 1024 B; byte lam*16 + i holds the E2M1 codes of columns
           128*ks + 32*g + 2*i (low nibble) and + 2*i + 1 (high nibble).
       ws (both): tile = 64 B; byte lam holds the E8M0 scale of the 32-block
           along K with index 4*ks + g (padding bytes 0).
"""
from __future__ import annotations

import numpy as np

from .quant import Quantized

TILE_M = 16
KSTEP = 128


def geometry(M: int, K: int):
    Mp = -(-M // TILE_M) * TILE_M
    Kp = -(-K // KSTEP) * KSTEP
    return Mp, Kp, Mp // TILE_M, Kp // KSTEP


def packed_bytes(fmt: str, M: int, K: int) -> tuple[int, int]:
    Mp, Kp, RT, KS = geometry(M, K)
    tiles = RT * KS
    if fmt == "int4":
        return tiles * 1024, tiles * 256
    if fmt == "int5":
        return tiles * 1024 + tiles * 256, tiles * 256
    if fmt == "int8":
        return tiles * 2048, tiles * 128
    if fmt == "nvfp4":
        return tiles * 1024, tiles * 128 + 16
    if fmt == "mxfp8":
        return tiles * 2048, tiles * 64
    if fmt == "mxfp4":
        return tiles * 1024, tiles * 64
    raise ValueError(fmt)


# slot e -> nibble index inside the int4 dword
_INT4_NIB = np.array([0, 4, 1, 5, 2, 6, 3, 7])


def _pad(a: np.ndarray, rows: int, cols: int) -> np.ndarray:
    out = np.zeros((rows, cols), dtype=a.dtype)
    out[: a.shape[0], : a.shape[1]] = a
    return out


def _codes_tiled(codes: np.ndarray, RT: int, KS: int) -> np.ndarray:
    """[Mp][Kp] -> [rt][ks][lane = s*16 + r][j][e]."""
    c = codes.reshape(RT, 16, KS, 4, 4, 8)          # rt, r, ks, j, s, e
    c = c.transpose(0, 2, 4, 1, 3, 5)               # rt, ks, s, r, j, e
    return c.reshape(RT, KS, 64, 4, 8)


def _untile_codes(t: np.ndarray, RT: int, KS: int) -> np.ndarray:
    c = t.reshape(RT, KS, 4, 16, 4, 8)              # rt, ks, s, r, j, e
    c = c.transpose(0, 3, 1, 4, 2, 5)               # rt, r, ks, j, s, e
    return c.reshape(RT * 16, KS * KSTEP)


# position of group j inside a row's scale record: groups 0, 2, 1, 3
_SCALE_POS = np.array([0, 2, 1, 3])       # pos(j) = 2*(j & 1) + (j >> 1)
_SCALE_J = np.argsort(_SCALE_POS)         # j stored at each position


def _scales_tiled(f: np.ndarray, RT: int, KS: int) -> np.ndarray:
    """per-group field [Mp][Kp/32] -> [rt][ks][r][pos]."""
    t = f.reshape(RT, 16, KS, 4).transpose(0, 2, 1, 3)
    return t[..., _SCALE_J]


def _untile_scales(t: np.ndarray, RT: int, KS: int) -> np.ndarray:
    t = t[..., _SCALE_POS]                # back to j order
    return t.transpose(0, 2, 1, 3).reshape(RT * 16, KS * 4)


def _nibble_dwords(t: np.ndarray, order: np.ndarray) -> np.ndarray:
    """[..., 8] codes (< 16) -> [...] uint32, code e in nibble order[e]."""
    sh = (4 * order).astype(np.uint32)
    return np.bitwise_or.reduce((t.astype(np.uint32) & np.uint32(0xF)) << sh, axis=-1)


def _dword_nibbles(w: np.ndarray, order: np.ndarray) -> np.ndarray:
    sh = (4 * order).astype(np.uint32)
    return ((w[..., None] >> sh) & np.uint32(0xF)).astype(np.uint8)


def _int5_place(j: int, e: int):
    """(dword, shift) of a whole 5-bit code, or None for pair 15."""
    P, h = 4 * j + (e >> 1), e & 1
    if P < 15:
        return P // 3, 16 * h + 5 * (P % 3)
    return None


def _int5_dwords(t: np.ndarray) -> np.ndarray:
    """codes [..., 4 (j), 8 (e)] (< 32) -> the lane's five dwords [..., 5]."""
    D = np.zeros(t.shape[:-2] + (5,), dtype=np.uint32)
    for j in range(4):
        for e in range(8):
            c = t[..., j, e].astype(np.uint32) & np.uint32(31)
            pl = _int5_place(j, e)
            if pl is not None:
                D[..., pl[0]] |= c << np.uint32(pl[1])
            else:
                for b in range(5):
                    D[..., b] |= ((c >> np.uint32(b)) & np.uint32(1)) << np.uint32(16 * (e & 1) + 15)
    return D


def _int5_codes(D: np.ndarray) -> np.ndarray:
    """the lane's five dwords [..., 5] -> codes [..., 4, 8]."""
    t = np.zeros(D.shape[:-1] + (4, 8), dtype=np.uint8)
    for j in range(4):
        for e in range(8):
            pl = _int5_place(j, e)
            if pl is not None:
                c = (D[..., pl[0]] >> np.uint32(pl[1])) & np.uint32(31)
            else:
                c = np.zeros(D.shape[:-1], dtype=np.uint32)
                for b in range(5):
                    c |= ((D[..., b] >> np.uint32(16 * (e & 1) + 15)) & np.uint32(1)) << np.uint32(b)
            t[..., j, e] = c.astype(np.uint8)
    return t


def pack(qz: Quantized) -> tuple[np.ndarray, np.ndarray]:
    """Logical fields -> (wq, ws) byte arrays in the device layout."""
    fmt, M, K = qz.fmt, qz.M, qz.K
    Mp, Kp, RT, KS = geometry(M, K)
    wq_n, ws_n = packed_bytes(fmt, M, K)
    if fmt in ("int4", "int5", "nvfp4"):
        codes = _pad(qz.codes.astype(np.uint8), Mp, Kp)
        t = _codes_tiled(codes, RT, KS)                              # rt ks lane j e
        order = _INT4_NIB if fmt != "nvfp4" else np.arange(8)
        nib = _nibble_dwords(t & np.uint8(0xF), order)               # rt ks lane j
        if fmt == "int5":
            D = _int5_dwords(t)                                       # rt ks lane 5
            wq = [D[..., :4].astype("<u4").tobytes(), D[..., 4].astype("<u4").tobytes()]
        else:
            wq = [nib.astype("<u4").tobytes()]
        wq = np.frombuffer(b"".join(wq), dtype=np.uint8).copy()
        if fmt == "nvfp4":
            sb = _pad(qz.sb.astype(np.uint8), Mp, Kp // 16)           # [Mp][8*KS]
            # block index 8ks + 2j + h  ->  [rt][ks][r][h][j]
            s5 = sb.reshape(RT, 16, KS, 4, 2).transpose(0, 2, 1, 4, 3)
            tail = np.zeros(16, dtype=np.uint8)
            tail[:4] = np.frombuffer(np.float32(qz.st).astype("<f4").tobytes(), dtype=np.uint8)
            ws = np.concatenate([s5.reshape(-1).astype(np.uint8), tail])
        else:
            d = _scales_tiled(_pad(qz.d, Mp, Kp // 32), RT, KS).astype(np.uint32)
            m = _scales_tiled(_pad(qz.m, Mp, Kp // 32), RT, KS).astype(np.uint32)
            ws = np.frombuffer((d | (m << np.uint32(16))).astype("<u4").tobytes(), dtype=np.uint8).copy()
    elif fmt == "int8":
        codes = _pad(qz.codes.astype(np.int8), Mp, Kp)
        t = _codes_tiled(codes, RT, KS)                              # rt ks lane j e
        t = t.reshape(RT, KS, 64, 2, 2, 8).transpose(0, 1, 3, 2, 4, 5)  # rt ks jhi lane jlo e
        wq = t.astype(np.int8).reshape(-1).view(np.uint8).copy()
        d = _scales_tiled(_pad(qz.d, Mp, Kp // 32), RT, KS)
        ws = np.frombuffer(d.astype("<u2").tobytes(), dtype=np.uint8).copy()
    elif fmt in ("mxfp8", "mxfp4"):
        codes = _pad(qz.codes.astype(np.uint8), Mp, Kp)
        if fmt == "mxfp8":
            t = codes.reshape(RT, 16, KS, 2, 4, 16).transpose(0, 2, 3, 4, 1, 5)      # rt ks h g r i
            wq = t.reshape(-1).copy()
        else:
            t = codes.reshape(RT, 16, KS, 4, 16, 2).transpose(0, 2, 3, 1, 4, 5)      # rt ks g r i pair
            wq = ((t[..., 0] & np.uint8(0xF)) | ((t[..., 1] & np.uint8(0xF)) << np.uint8(4))).reshape(-1).copy()
        e = _pad(qz.e.astype(np.uint8), Mp, Kp // 32)
        ws = e.reshape(RT, 16, KS, 4).transpose(0, 2, 3, 1).reshape(-1).copy()         # rt ks g r
    else:
        raise ValueError(fmt)
    assert wq.size == wq_n and ws.size == ws_n, (wq.size, wq_n, ws.size, ws_n)
    return wq, ws


def unpack(fmt: str, M: int, K: int, wq: np.ndarray, ws: np.ndarray) -> Quantized:
    """(wq, ws) device bytes -> logical fields (padding dropped)."""
    Mp, Kp, RT, KS = geometry(M, K)
    wq_n, ws_n = packed_bytes(fmt, M, K)
    wq = np.asarray(wq, dtype=np.uint8)
    ws = np.asarray(ws, dtype=np.uint8)
    if wq.size != wq_n or ws.size != ws_n:
        raise ValueError("buffer sizes do not match the geometry")
    tiles = RT * KS
    if fmt in ("int4", "int5", "nvfp4"):
        nib = wq[: tiles * 1024].view("<u4").reshape(RT, KS, 64, 4)
        if fmt == "int5":
            D = np.concatenate([nib, wq[tiles * 1024:].view("<u4").reshape(RT, KS, 64, 1)], axis=-1)
            t = _int5_codes(D)                                        # rt ks lane j e
        else:
            order = _INT4_NIB if fmt != "nvfp4" else np.arange(8)
            t = _dword_nibbles(nib, order)                            # rt ks lane j e
        codes = _untile_codes(t, RT, KS)[:M, :K]
        if fmt == "nvfp4":
            s5 = ws[: tiles * 128].reshape(RT, KS, 16, 2, 4)              # rt ks r h j
            sb = s5.transpose(0, 2, 1, 4, 3).reshape(Mp, Kp // 16)[:M, : K // 16]
            st = ws[tiles * 128: tiles * 128 + 4].view("<f4")[0]
            return Quantized(fmt, M, K, codes.copy(), sb=sb.copy(), st=np.float32(st))
        dm = ws.view("<u4").reshape(RT, KS, 16, 4)
        dm = _untile_scales(dm, RT, KS)[:M, : K // 32]
        d = (dm & np.uint32(0xFFFF)).astype(np.uint16)
        m = (dm >> np.uint32(16)).astype(np.uint16)
        return Quantized(fmt, M, K, codes.copy(), d=d, m=m)
    if fmt in ("mxfp8", "mxfp4"):
        if fmt == "mxfp8":
            codes = wq.reshape(RT, KS, 2, 4, 16, 16).transpose(0, 4, 1, 2, 3, 5).reshape(Mp, Kp)
        else:
            b = wq.reshape(RT, KS, 4, 16, 16)                                        # rt ks g r i
            t = np.stack([b & np.uint8(0xF), b >> np.uint8(4)], axis=-1)             # rt ks g r i pair
            codes = t.transpose(0, 3, 1, 2, 4, 5).reshape(Mp, Kp)
        e = ws.reshape(RT, KS, 4, 16).transpose(0, 3, 1, 2).reshape(Mp, Kp // 32)
        return Quantized(fmt, M, K, codes[:M, :K].copy(), e=e[:M, : K // 32].copy())
    if fmt == "int8":
        t = wq.view(np.int8).reshape(RT, KS, 2, 64, 2, 8).transpose(0, 1, 3, 2, 4, 5)
        codes = _untile_codes(t.reshape(RT, KS, 64, 4, 8), RT, KS)[:M, :K]
        d = _untile_scales(ws.view("<u2").reshape(RT, KS, 16, 4), RT, KS)[:M, : K // 32]
        return Quantized(fmt, M, K, codes.copy(), d=d.astype(np.uint16))
    raise ValueError(fmt)
