// Device helpers shared by the gfx950 kernels: MFMA wrappers, buffer
// resources for direct-to-LDS loads, counted waits, the clamped SwiGLU and
// the 4-bit block decode.
#pragma once

#include "moe_internal.h"

namespace moe {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ floatx16 mfma32(half8 a, half8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16(half8 a, half8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16f32(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <class V>
__device__ __forceinline__ V as_v8(uint4 u) { return __builtin_bit_cast(V, u); }

__device__ __forceinline__ uint4 ldg16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Raw buffer resource over [base, base + bytes): scalar registers hold the
// descriptor, lanes pass 32-bit byte offsets.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                            uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)bytes, 0x00020000);
}

// s_waitcnt with vmcnt(N) only (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// vmcnt(N) and lgkmcnt(0) together.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);
}

// Work-item order for a persistent grid of G blocks, in rounds of G items:
// the blocks of one XCD (hardware block ids b = x mod 8) take one contiguous
// run of the round's items, so items that share operands (the column blocks
// of one expert group) run on one XCD and share its L2. A round of R < G
// items gives XCD x floor(R / 8) or one more. Returns the item of block b in
// the round starting at rb0, or -1 if b sits this round out.
__device__ __forceinline__ int xcd_item(int rb0, int b, int G, int n_items) {
  const int R = min(G, n_items - rb0);
  if (G & 7) return b < R ? rb0 + b : -1;
  const int x = b & 7, m = b >> 3;
  const int q = R >> 3, r = R & 7;
  if (m >= q + (x < r ? 1 : 0)) return -1;
  return rb0 + x * q + min(x, r) + m;
}

// h = silu(min(g, c)) * clamp(u, -c, c); c <= 0: plain silu(g) * u.
// silu(g) = g / (1 + e^-g) with the hardware's 2^x and reciprocal (about
// one ulp each): the epilogues evaluate it for every (pair, feature), and a
// libm-accurate exp there costs more time than the tile's last stages.
// The clamps are one v_med3_f32 each (c <= 0 means no clamp: the bound
// becomes +inf, which the compiler folds once per kernel, not per value).
__device__ __forceinline__ float swiglu(float g, float u, float c) {
  const float cl = c > 0.f ? c : __builtin_inff();
  g = __builtin_amdgcn_fmed3f(g, -__builtin_inff(), cl);
  u = __builtin_amdgcn_fmed3f(u, -cl, cl);
  const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896340736f);
  return g * __builtin_amdgcn_rcpf(1.f + e) * u;
}

// The 8 nibbles of a word (low nibble first) as 4 pairs of fp16 bit
// patterns 0x6400 | v (the fp16 value 1024 + v, exactly): byte-interleave
// the low and high nibbles into [v0 v1 v2 v3], [v4 v5 v6 v7], then spread
// each byte to the low byte of a 16-bit half whose high byte v_perm takes
// from a register of 0x64 bytes (two selects a pair, no OR).
// flip: XORed into every isolated nibble (8 turns a two's-complement nibble
// q into q + 8; the mask and the flip make one three-input logic op).
__device__ __forceinline__ void unpack_nibbles(uint32_t x, uint32_t out[4],
                                               uint32_t flip = 0u) {
  const uint32_t lo = (x & 0x0F0F0F0Fu) ^ flip;          // v0 v2 v4 v6
  const uint32_t hi = ((x >> 4) & 0x0F0F0F0Fu) ^ flip;   // v1 v3 v5 v7
  const uint32_t p0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // v0 v1 v2 v3
  const uint32_t p1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // v4 v5 v6 v7
  const uint32_t c = 0x64646464u;
  out[0] = __builtin_amdgcn_perm(c, p0, 0x04010400u);   // [v0, 0x64, v1, 0x64]
  out[1] = __builtin_amdgcn_perm(c, p0, 0x04030402u);
  out[2] = __builtin_amdgcn_perm(c, p1, 0x04010400u);
  out[3] = __builtin_amdgcn_perm(c, p1, 0x04030402u);
}

// 8 consecutive 4-bit values (one 32-bit word, low nibble first) times
// their block scale, as 8 fp16: fp16 bits 0x6400 | v encode 1024 + v
// exactly, v = nibble ^ 8 = q + 8; subtracting 1032 leaves the signed value
// q exactly, and one fp16 multiply gives fp16_rne(q * s).
__device__ __forceinline__ half8 dequant_word(uint32_t word, _Float16 s) {
  const half2v s2 = {s, s};
  const half2v off = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  uint32_t pr[4];
  unpack_nibbles(word, pr, 0x08080808u);
  half8 out;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    half2v h = __builtin_bit_cast(half2v, pr[b]);
    h = (h + off) * s2;
    out[2 * b] = h[0];
    out[2 * b + 1] = h[1];
  }
  return out;
}

// 32 consecutive 4-bit values (16 bytes) of one block, as 4 x 8 fp16.
__device__ __forceinline__ void dequant32(uint4 raw, _Float16 s, half8 out[4]) {
  out[0] = dequant_word(raw.x, s);
  out[1] = dequant_word(raw.y, s);
  out[2] = dequant_word(raw.z, s);
  out[3] = dequant_word(raw.w, s);
}

// 4-bit weight formats. FMT 0 (MOE_Q4B32): two's-complement nibbles, one
// fp16 scale per 32 K values, value q * s. FMT 1 / 2 (MOE_Q4A32 / Q4A64):
// unsigned nibbles, an fp16 (scale, bias) pair per 32 / 64 K values stored
// as one 32-bit word (scale in the low half), value q * s + b: the affine
// 4-bit groups of the MLX checkpoints TensorFold PR #1607 serves.
template <int FMT> struct Q4F {
  static constexpr int kGroup = FMT == 2 ? 64 : 32;   // K values per parameter
  static constexpr int kPB = FMT == 0 ? 2 : 4;         // bytes per parameter
};

// Parameters of a lane's 32 * KH consecutive K values from k0 (k0 a
// multiple of 32 * KH) of one weight row whose parameters start at prow.
struct Q4P { uint32_t w[2]; };
template <int FMT, int KH>
__device__ __forceinline__ Q4P load_q4p(const char* prow, int k0) {
  Q4P p{{0u, 0u}};
  if constexpr (FMT == 0) {
    if constexpr (KH == 2)   // two adjacent fp16 scales, 4-byte aligned
      p.w[0] = *reinterpret_cast<const uint32_t*>(prow + (k0 / 32) * 2);
    else
      p.w[0] = *reinterpret_cast<const uint16_t*>(prow + (k0 / 32) * 2);
  } else if constexpr (FMT == 1) {
    if constexpr (KH == 2) {
      const uint2 v = *reinterpret_cast<const uint2*>(prow + (k0 / 32) * 4);
      p.w[0] = v.x;
      p.w[1] = v.y;
    } else {
      p.w[0] = *reinterpret_cast<const uint32_t*>(prow + (k0 / 32) * 4);
    }
  } else {
    p.w[0] = *reinterpret_cast<const uint32_t*>(prow + (k0 / 64) * 4);
  }
  return p;
}
// the parameter of the lane's 32-value block h
template <int FMT>
__device__ __forceinline__ uint32_t q4p_block(const Q4P& p, int h) {
  if constexpr (FMT == 0) return (p.w[0] >> (16 * h)) & 0xFFFFu;
  else if constexpr (FMT == 1) return p.w[h];
  else return p.w[0];
}

// 8 consecutive unsigned 4-bit values (low nibble first) as fp16
// q * s + b: 0x6400 | q encodes 1024 + q exactly, subtracting 1024 leaves q,
// and one fp16 fma rounds q * s + b once.
__device__ __forceinline__ half8 dequant_word_affine(uint32_t word, uint32_t sb) {
  const _Float16 sc = __builtin_bit_cast(_Float16, (uint16_t)(sb & 0xFFFFu));
  const _Float16 bi = __builtin_bit_cast(_Float16, (uint16_t)(sb >> 16));
  const half2v s2 = {sc, sc};
  const half2v b2 = {bi, bi};
  const half2v off = {(_Float16)-1024.0f, (_Float16)-1024.0f};
  uint32_t pr[4];
  unpack_nibbles(word, pr);
  half8 out;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    half2v h = __builtin_bit_cast(half2v, pr[b]) + off;
    h = __builtin_elementwise_fma(h, s2, b2);
    out[2 * b] = h[0];
    out[2 * b + 1] = h[1];
  }
  return out;
}

template <int FMT>
__device__ __forceinline__ half8 dequant_word_f(uint32_t word, uint32_t param) {
  if constexpr (FMT == 0)
    return dequant_word(word, __builtin_bit_cast(_Float16, (uint16_t)param));
  else
    return dequant_word_affine(word, param);
}

template <int FMT>
__device__ __forceinline__ void dequant32_f(uint4 raw, uint32_t param, half8 out[4]) {
  out[0] = dequant_word_f<FMT>(raw.x, param);
  out[1] = dequant_word_f<FMT>(raw.y, param);
  out[2] = dequant_word_f<FMT>(raw.z, param);
  out[3] = dequant_word_f<FMT>(raw.w, param);
}

// Per-pair outputs of the down projection: fp16 when the layer computes in
// fp16 (no range or precision is lost against its fp16 intermediate), f32
// otherwise (bf16's 8-bit significand would cost the output its tolerance).
template <class S> struct YPairOf { using T = float; };
template <> struct YPairOf<_Float16> { using T = _Float16; };

template <class Y>
__device__ __forceinline__ void store_y4(void* base, size_t idx, float a,
                                         float b, float c, float d) {
  if constexpr (sizeof(Y) == 2) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    h4 v = {(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};
    *reinterpret_cast<h4*>(reinterpret_cast<_Float16*>(base) + idx) = v;
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + idx) = float4{a, b, c, d};
  }
}

template <class Y>
__device__ __forceinline__ void store_y1(void* base, size_t idx, float a) {
  reinterpret_cast<Y*>(base)[idx] = (Y)a;
}

}  // namespace moe
