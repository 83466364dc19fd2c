// fa_dropout.hpp -- dropout of the attention weights inside the fused kernels,
// regenerated in the backward pass from the generator state instead of being
// stored ("como funciona", tonho.wtf digest; algorithm paragraph of the
// agihunt.info summary).
//
// The mask.  Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random
// Numbers: As Easy as 1, 2, 3", SC 2011): a 4-word counter and a 2-word key;
// each of 10 rounds multiplies counter words 0 and 2 by two fixed 32-bit
// multipliers and rebuilds the counter from the high and low product halves,
// the other two words and the key; the key is advanced by two fixed Weyl
// increments between rounds.  One evaluation with counter
// (j / 4, i / 4, head, offset) covers the 4 x 4 block of (query i, key j)
// pairs: word i mod 4, byte j mod 4 decides pair (i, j), kept iff the byte is
// >= t8 = floor(256 p).  Kept weights are scaled by 256 / (256 - t8); the
// kernels apply that scale once to their finished outputs.
//
// Work split.  A wave's 32 x 32 block of pairs holds 64 such 4 x 4 blocks, one
// per lane: every lane evaluates the generator once, and a quad of lanes
// (4 consecutive queries in the forward / dQ layout, 4 consecutive keys in the
// dK/dV layout) swaps words through a 1280-byte LDS area of the wave so that
// each lane ends up with the bytes of its own registers.  No evaluation is
// repeated.
#pragma once

#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {

constexpr int kDropLdsPerWave = 16 * 20 * 4;  // 16 quads x 20 words (16 + 4 padding)

__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                              uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)c0 * 0xD2511F53u;
    const uint64_t p1 = (uint64_t)c2 * 0xCD9E8D57u;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return u32x4{c0, c1, c2, c3};
}

// Quad exchange: lane (quad q, position a) supplies x[k], k = 0..3, and
// receives y[k] = x[a] of the quad's lane k (a 4 x 4 transpose across the
// quad).  xlds: this wave's kDropLdsPerWave bytes.
__device__ __forceinline__ u32x4 quad_transpose(u32x4 x, char* xlds, int lane) {
  uint32_t* base = (uint32_t*)xlds + (lane >> 2) * 20;
  const int a = lane & 3;
#pragma unroll
  for (int k = 0; k < 4; ++k) base[k * 4 + a] = x[k];
  return *(const u32x4*)(base + a * 4);
}

// Forward / dQ layout (one query per lane, registers along keys).  For the
// block of keys key0 .. key0+31 and queries query0 .. query0+31 (both
// multiples of 4), returns w with: byte e of w[rr] is the generator byte of
// (this lane's query, the key of register rr * 4 + e), that key being
// key0 + rr * 8 + 4 * (lane / 32) + e.
__device__ __forceinline__ u32x4 drop_bytes_query_lanes(const DropParams& d, uint32_t head,
                                                        int key0, int query0, char* xlds,
                                                        int lane) {
  const int g = lane >> 5, l32 = lane & 31, a = l32 & 3;
  // this lane evaluates key group rr = a of its quad's 4 queries
  const u32x4 x = philox4x32_10((uint32_t)(key0 >> 2) + 2 * a + g,
                                (uint32_t)(query0 >> 2) + (l32 >> 2), head, d.offset, d.k0, d.k1);
  return quad_transpose(x, xlds, lane);
}

// dK/dV layout (one key per lane, registers along queries).  For keys
// key0 .. key0+31 and queries query0 .. query0+31, returns w with: byte e of
// w[rr] is the generator byte of (the query of register rr * 4 + e, this
// lane's key), that query being query0 + rr * 8 + 4 * (lane / 32) + e.
__device__ __forceinline__ u32x4 drop_bytes_key_lanes(const DropParams& d, uint32_t head, int key0,
                                                      int query0, char* xlds, int lane) {
  const int g = lane >> 5, l32 = lane & 31, a = l32 & 3;
  // this lane evaluates query group rr = a for its quad's 4 keys
  const u32x4 x = philox4x32_10((uint32_t)(key0 >> 2) + (l32 >> 2),
                                (uint32_t)(query0 >> 2) + 2 * a + g, head, d.offset, d.k0, d.k1);
  // byte transpose: t[b] holds byte b (key j mod 4 = b) of x[0..3] (rows 0..3)
  const uint32_t lo01 = __builtin_amdgcn_perm(x[1], x[0], 0x05010400u);
  const uint32_t lo23 = __builtin_amdgcn_perm(x[3], x[2], 0x05010400u);
  const uint32_t hi01 = __builtin_amdgcn_perm(x[1], x[0], 0x07030602u);
  const uint32_t hi23 = __builtin_amdgcn_perm(x[3], x[2], 0x07030602u);
  u32x4 t;
  t[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
  t[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
  t[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
  t[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
  return quad_transpose(t, xlds, lane);
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Keep masks of bytes 2h and 2h+1 of w as two 16-bit halves (0xFFFF kept,
// 0x0000 dropped), to AND with a packed pair of 16-bit weights.  bias holds
// 0x8000 - t8 in both halves: byte + bias has bit 15 set iff byte >= t8.
__device__ __forceinline__ uint32_t keep_pair_mask(uint32_t w, int h, uint32_t bias) {
  const uint32_t spread = __builtin_amdgcn_perm(0u, w, h ? 0x0c030c02u : 0x0c010c00u);
  const uint32_t sum = __builtin_bit_cast(
      uint32_t, __builtin_bit_cast(u16x2, spread) + __builtin_bit_cast(u16x2, bias));
  return __builtin_amdgcn_perm(0u, sum, 0x09090808u);  // replicate bits 15 and 31
}

__device__ __forceinline__ bool keep_byte(uint32_t w, int e, uint32_t t8) {
  return ((w >> (8 * e)) & 0xFFu) >= t8;
}

}  // namespace fa
