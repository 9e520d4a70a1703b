// Packed-weight geometry shared by the host packer and the device kernels.
//
// The subject pages only say that engines repack checkpoints into their own
// layout (memra page, model notes) and pack 4-bit codes as nibbles along K.
// This layout is built for a 64-lane CDNA wave: one 16-byte load per lane
// fetches one contiguous 1 KiB tile of 16 rows x 128 columns of 4-bit codes,
// and the lane's bytes are exactly the B operand of a 16x16x32 bf16 MFMA.
//
//   Mp = M rounded up to 16, Kp = K rounded up to 128; padding is weight 0.
//   RT = Mp/16 row tiles, KS = Kp/128 k-steps, tile index tau = rt*KS + ks.
//   Lane lam: r = lam % 16 (row 16*rt + r), s = lam / 16; group j in [0,4),
//   slot e in [0,8): column k = 128*ks + 32*j + 8*s + e.
//
//   int4  wq tile 1024 B: lane's 16 B at lam*16, dword j = group j, slot e in
//         nibble (e even ? e/2 : 4 + e/2).  ws tile 256 B: row r's 16 B at
//         r*16, group j's dword (d | m<<16, fp16 bits) at position
//         2*(j&1) + (j>>1).
//   int5  wq = plane A of 1024 B tiles (lane's dwords D0..D3 at lam*16) then
//         plane B of 256 B tiles (lane's dword D4 at lam*4). The lane's 32
//         codes form 16 pairs P = 4*j + (e>>1), half h = e & 1 (slot e of
//         group j). For P < 15 the 5-bit code is bits 16*h + 5*(P%3) .. +4
//         of dword D(P/3); for P = 15, code bit b is bit 16*h + 15 of D(b).
//         ws as int4.
//   int8  wq tile 2048 B: byte (j>>1)*1024 + lam*16 + (j&1)*8 + e.
//         ws tile 128 B: fp16 d at r*8 + 2*(2*(j&1) + (j>>1)).
//   nvfp4 wq tile 1024 B: byte lam*16 + 4*j + e/2, low nibble even e.
//         ws tile 128 B: E4M3 of 16-block 8*ks + 2*j + h at r*8 + 4*h + j;
//         then the fp32 tensor scale at RT*KS*128, padded to 16 B.
//
// MX formats take the register layout of gfx950's block-scaled 16x16x128
// MFMA instead (lane lam: row 16*rt + lam % 16, g = lam / 16), so each lane's
// loads are its B operand as is:
//   mxfp8 wq tile 2048 B: byte h*1024 + lam*16 + i = E4M3 code of column
//         128*ks + 64*h + 16*g + i (h < 2, i < 16).
//   mxfp4 wq tile 1024 B: byte lam*16 + i = E2M1 codes of columns
//         128*ks + 32*g + 2*i (low nibble) and 2*i + 1 (high nibble).
//   ws (both) tile 64 B: byte lam = E8M0 scale of row 16*rt + lam % 16,
//         32-block 4*ks + g.
#pragma once
#include <stdint.h>
#include <stddef.h>

namespace qg {

enum Fmt : int { INT4 = 1, INT5 = 2, INT8 = 3, NVFP4 = 4, MXFP4 = 5, MXFP8 = 6 };

struct Geom {
  int64_t M, K, Mp, Kp, RT, KS;
  size_t wq_bytes, ws_bytes;
  size_t hi_offset;      // int5: byte offset of the hi-bit plane in wq
  size_t st_offset;      // nvfp4: byte offset of the tensor scale in ws
};

inline bool geom(int fmt, int64_t M, int64_t K, Geom* g) {
  if (M < 1 || K < 32 || (K % 32) != 0) return false;
  g->M = M;
  g->K = K;
  g->Mp = (M + 15) / 16 * 16;
  g->Kp = (K + 127) / 128 * 128;
  g->RT = g->Mp / 16;
  g->KS = g->Kp / 128;
  const size_t tiles = (size_t)g->RT * (size_t)g->KS;
  g->hi_offset = 0;
  g->st_offset = 0;
  switch (fmt) {
    case INT4: g->wq_bytes = tiles * 1024; g->ws_bytes = tiles * 256; break;
    case INT5: g->wq_bytes = tiles * 1280; g->ws_bytes = tiles * 256; g->hi_offset = tiles * 1024; break;
    case INT8: g->wq_bytes = tiles * 2048; g->ws_bytes = tiles * 128; break;
    case NVFP4: g->wq_bytes = tiles * 1024; g->ws_bytes = tiles * 128 + 16; g->st_offset = tiles * 128; break;
    case MXFP4: g->wq_bytes = tiles * 1024; g->ws_bytes = tiles * 64; break;
    case MXFP8: g->wq_bytes = tiles * 2048; g->ws_bytes = tiles * 64; break;
    default: return false;
  }
  return true;
}

inline int scale_pos(int j) { return 2 * (j & 1) + (j >> 1); }

}  // namespace qg
