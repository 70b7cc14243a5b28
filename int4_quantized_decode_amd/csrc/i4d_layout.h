// i4d_layout.h - device data layouts of the INT4 decode block (gfx950).
//
// Weights.  A packed projection has Np rows (Np = N, or 2N for gate/up) and K
// input channels.  Rows are cut into 16-row strips and K into 128-wide groups
// (the quantization groups).  One (strip, group) "atom" is 1 KiB of codes:
// 64 lanes x 16 bytes, arranged for a 64-wide wavefront:
//
//   lane l = 16*j + r   (r = row in strip, j = 0..3)
//   lane bytes = 4 dwords, dword kb (0..3) holds the 8 codes of row r at
//   k = 128*g + 32*kb + 8*j + e, e = 0..7
//
// which is exactly the A operand a lane holds for the 16x16x32 bf16 MFMA
// (row = lane % 16, k = 8*(lane/16) .. +7) over the four K=32 steps of a
// group, and also a 16-byte coalesced load for the VALU GEMV.  Inside a dword
// the nibble slot of code e is sigma(e) = 4*(e&1) + (e>>1), i.e. slots hold
// e = 0,2,4,6,1,3,5,7: masking the dword (>> 4i) with 0x000F000F yields the
// bf16/fp16 pair (e = 2i, 2i+1) in one v_and_or_b32.  Nibbles are u = q + 8.
//
// Scales: fp16, [strip][group/8][row 16][group%8], the group count padded to
// a multiple of 8 with zeros: one 16-byte load gives a row 8 groups' scales.
//
// Row order inside strips: PLAIN keeps the natural order.  QKV pairs the RoPE
// partners: strip s of a head holds rows 8s..8s+7 then hd/2+8s..hd/2+8s+7.
// GATE_UP holds gate rows 8t..8t+7 then up rows 8t..8t+7 in strip t.
//
// KV cache.  Slot e = row_base[r]*n_kv + j*cap_r + t (cap_r % 32 == 0).
//   keys:   hd/2 bytes per slot, laid out like one weight atom row: chunk jj
//           (16 B for hd=128, 8 B for hd=64) holds dwords kb with channels
//           32*kb + 8*jj + e (same nibble slots as weights).  A 16-token
//           tile is the MFMA A operand (row = token) for q.k.
//   values: per 32-token block (slots 32b..32b+31 of one (row, head)),
//           4*hd dwords; dword (jj, c16, cb) at index jj*hd + c16*(hd/16) + cb
//           holds channel 16*cb + c16 of the 8 tokens of "slot group" jj:
//           e = 0..3 -> token 4*jj + e, e = 4..7 -> token 16 + 4*jj + e - 4,
//           nibble slot sigma(e).  This is the MFMA A operand of V^T for the
//           P.V product with token-slots as the reduction axis.
//   scales: fp16 per slot.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace i4d {

constexpr int kGroup = 128;
constexpr int kStrip = 16;
constexpr int kAtomBytes = 1024;
constexpr int kVBlock = 32;

inline constexpr int nibble_slot(int e) { return 4 * (e & 1) + (e >> 1); }

// E4M3 weights (the FP8 decode-weight variant): one byte per weight, the
// same strips, groups and scales; an atom (strip, group) is 2 KiB: lane
// l = 16*j + r holds 32 bytes, byte 8*kb + e = the code of row r at
// k = 128*g + 32*kb + 8*j + e (kb = 0..3, e = 0..7), i.e. the four bf16 MFMA
// A operands of the group in k order once decoded, two 16-byte loads.
constexpr int kAtomBytesE4M3 = 2048;

inline size_t e4m3_code_offset(int p, int k, int K) {
  int t = p / kStrip, r = p % kStrip, g = k / kGroup, kk = k % kGroup;
  int kb = kk / 32, j = (kk % 32) / 8, e = kk % 8;
  return (((size_t)t * (K / kGroup) + g) * 64 + 16 * j + r) * 32 + kb * 8 + e;
}

inline int groups_of(int K) { return K / kGroup; }
inline int g8_of(int K) { return (K / kGroup + 7) / 8; }

inline size_t packed_code_bytes(int Np, int K) { return (size_t)Np * (size_t)K / 2; }
// scales: fp16 [strip][group][16 rows], 32 bytes per atom
inline size_t packed_scale_elems(int Np, int K) {
  return (size_t)(Np / kStrip) * (size_t)groups_of(K) * kStrip;
}

// byte offset of code (packed row p, k) and the nibble slot inside it
inline size_t code_byte_offset(int p, int k, int K, int* nib_hi) {
  int t = p / kStrip, r = p % kStrip, g = k / kGroup, kk = k % kGroup;
  int kb = kk / 32, j = (kk % 32) / 8, e = kk % 8;
  int lane = 16 * j + r;
  int slot = nibble_slot(e);
  *nib_hi = slot & 1;
  return (((size_t)t * groups_of(K) + g) * 64 + lane) * 16 + kb * 4 + slot / 2;
}

inline size_t scale_index(int p, int g, int K) {
  int t = p / kStrip, r = p % kStrip;
  return ((size_t)t * groups_of(K) + g) * kStrip + r;
}

// packed row -> logical row for each kind (QKV needs head_dim)
inline int qkv_logical_row(int p, int hd) {
  int t = p / kStrip, i = p % kStrip;
  int per_head = hd / kStrip;
  int head = t / per_head, sp = t % per_head;
  int c = (i < 8) ? (8 * sp + i) : (hd / 2 + 8 * sp + (i - 8));
  return head * hd + c;
}

// key slot: byte offset of channel c within a token's hd/2 bytes
inline int key_byte_in_slot(int c, int hd, int* nib_hi) {
  int kb = c / 32, jj = (c % 32) / 8, e = c % 8;
  int slot = nibble_slot(e);
  *nib_hi = slot & 1;
  int chunk = (hd == 128) ? 16 : 8;
  return jj * chunk + kb * 4 + slot / 2;
}

// value block: dword index and nibble slot of (token w in block, channel c)
inline int value_dword_in_block(int w, int c, int hd, int* slot) {
  int jj, e;
  if (w < 16) { jj = w / 4; e = w % 4; } else { jj = (w - 16) / 4; e = 4 + (w - 16) % 4; }
  *slot = nibble_slot(e);
  return jj * hd + (c % 16) * (hd / 16) + c / 16;
}

}  // namespace i4d
