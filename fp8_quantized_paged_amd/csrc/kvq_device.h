// Device helpers shared by the kvq kernels (gfx950 only).
//
// e4m3 here is the OCP "e4m3fn" format the pages store the cache in: sign, 4
// exponent bits (bias 7), 3 mantissa bits, max 448, NaN 0x7F/0xFF, no infinity.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kPage = 16;
constexpr int kWave = 64;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) {
  return __uint_as_float(h << 16);
}

// float32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) | 0x40u) & 0xFFFFu;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Round-to-nearest-even, saturating float32 -> e4m3 encoder, without branches.
// NaN -> 0x7F | sign; |x| >= 448 (and inf) -> 0x7E | sign; sign of zero kept.
// Normal range [2^-6, 448): keep 3 of the 23 fraction bits, ties to even (a carry may
// bump the exponent); e4m3 exponent = float32 exponent - 120.  Below 2^-6 the grid
// is n * 2^-9, n = 0..8: |x| * 2^9 is exact and rint rounds half to even.
// (Also built for the host so it can be checked exhaustively on a CPU.)
__host__ __device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  const uint32_t normal = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
  // the clamp keeps the conversion defined for inputs that take another branch
  const float scaled = __builtin_fminf(__builtin_bit_cast(float, a) * 512.0f, 8.0f);
  const uint32_t sub = (uint32_t)__builtin_rintf(scaled);
  uint32_t code = a >= 0x3C800000u ? normal : sub;  // 2^-6
  code = a >= 0x43E00000u ? 0x7Eu : code;           // 448
  code = a > 0x7F800000u ? 0x7Fu : code;            // NaN
  return code | sign;
}

// Code of x at scale s: encode(fl32(x / s)) with IEEE division; a NaN quotient
// takes the sign of x (the sign of a NaN produced by division is not fixed).
__host__ __device__ __forceinline__ uint32_t e4m3_quantize(float x, float s) {
  const float q = x / s;
  if (q != q) return 0x7Fu | ((__builtin_bit_cast(uint32_t, x) >> 24) & 0x80u);
  return e4m3_encode(q);
}

// Codes of x0 / s and x1 / s (IEEE division) on gfx950's converter, bytes 0 and 1 of
// the result: the quotient is clamped to +-448 first (the converter itself does not
// saturate) and a NaN quotient takes 0x7F | sign of x.  The converter's round to nearest
// even equals e4m3_encode on every non-NaN float32 input (all 2^32 patterns checked on
// an MI355X), so the codes equal e4m3_quantize's; it does two values in one instruction
// where the integer encoder takes about a dozen per value.  x / 1 is x, so a unit scale
// skips the division.
__device__ __forceinline__ uint32_t e4m3_codes2(float q0, float q1, float x0, float x1) {
  const float c0 = __builtin_amdgcn_fmed3f(q0, -448.0f, 448.0f);
  const float c1 = __builtin_amdgcn_fmed3f(q1, -448.0f, 448.0f);
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false) & 0xFFFFu;
  if (q0 != q0) w = (w & 0xFF00u) | 0x7Fu | ((__float_as_uint(x0) >> 24) & 0x80u);
  if (q1 != q1) w = (w & 0x00FFu) | ((0x7Fu | ((__float_as_uint(x1) >> 24) & 0x80u)) << 8);
  return w;
}
__device__ __forceinline__ uint32_t e4m3_quantize2(float x0, float x1, float s) {
  if (s == 1.0f) return e4m3_codes2(x0, x1, x0, x1);
  return e4m3_codes2(x0 / s, x1 / s, x0, x1);
}
// Four codes (bytes 0..3) of x[0..3] / s.
__device__ __forceinline__ uint32_t e4m3_quantize4(const float* x, float s) {
  return e4m3_quantize2(x[0], x[1], s) | (e4m3_quantize2(x[2], x[3], s) << 16);
}

// x / s for the values of one per-token-head row, s = fl32(amax / 448), from a
// reciprocal r of s (once per row) and two fused multiply-adds per value: q0 = x r, the residual
// e = q0 s - x (exact), q = q0 - e r (Markstein's correction step).  Negating the
// residual rather than the product keeps the sign of zero: a residual that vanishes is
// +0, and q0 - (+0) r leaves q0 (-0 for x = -0) unchanged; otherwise it is exactly the
// negated residual x - q0 s.  Where it is used -- 2^-100 <= amax < inf, |x| <= amax --
// its e4m3 code equals that of the IEEE quotient for every bf16 x and every bf16 amax,
// with r = RN(1 / s) and with r from the hardware reciprocal (all such pairs checked on
// an MI355X; the quotients themselves differ in about 0.1% of them, never across an
// e4m3 rounding boundary).  Rows with smaller, infinite or NaN maxima take the
// division (row_quot_fast false).
__device__ __forceinline__ bool row_quot_fast(uint32_t amax_bits) {
  return amax_bits >= 0x0D800000u && amax_bits < 0x7F800000u;  // [2^-100, inf)
}
__device__ __forceinline__ float row_quot(float x, float s, float r) {
  const float q0 = x * r;
  return __builtin_fmaf(-__builtin_fmaf(q0, s, -x), r, q0);
}
// Four codes (bytes 0..3) of a per-token-head row's x[0..3] / s (r from row_scale when
// fast).  On a fast row every quotient is finite with |q| <= 448 (1 + 2^-22), below 464,
// up to which the converter rounds to +-448 (checked for every float in [448, 464] of
// both signs): no clamp and no NaN fix-up.
__device__ __forceinline__ uint32_t e4m3_quantize4_row(const float* x, float s, float r,
                                                       bool fast) {
  if (!fast) return e4m3_quantize4(x, s);
  float q[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) q[j] = row_quot(x[j], s, r);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], (int)lo, true);
}

// Row maxima of |x| for a per-token-head row of K and one of V, held by `lanes`
// consecutive lanes (8 bf16 values of each per lane, power-of-two lanes): as bf16
// magnitude bit patterns, K in bits 0-15 and V in bits 16-31, reduced with packed 16-bit
// integer maxima (magnitude bits order like the values, NaN above infinity, so a NaN
// propagates), one shuffle chain for both.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a),
                                                                __builtin_bit_cast(u16x2_t, b)));
}
template <int kLanes>
__device__ __forceinline__ uint32_t row_amax_bf16_kv(uint4 kw, uint4 vw) {
  constexpr uint32_t kMag = 0x7FFF7FFFu;
  const uint32_t mk = pk_max_u16(pk_max_u16(kw.x & kMag, kw.y & kMag), pk_max_u16(kw.z & kMag, kw.w & kMag));
  const uint32_t mv = pk_max_u16(pk_max_u16(vw.x & kMag, vw.y & kMag), pk_max_u16(vw.z & kMag, vw.w & kMag));
  // (K lo, V lo) and (K hi, V hi) pairs, then their maximum
  uint32_t m = pk_max_u16(__builtin_amdgcn_perm(mv, mk, 0x05040100u),
                          __builtin_amdgcn_perm(mv, mk, 0x07060302u));
#pragma unroll
  for (int o = kLanes / 2; o >= 1; o >>= 1) m = pk_max_u16(m, (uint32_t)__shfl_xor((int)m, o));
  return m;
}

// Per-token-head scale from the magnitude bits of the row maximum.
__device__ __forceinline__ float scale_from_amax_bits(uint32_t amax_bits) {
  if (amax_bits == 0u) return 1.0f;
  return __uint_as_float(amax_bits) / 448.0f;
}
// A row's scale s = fl32(amax / 448) and, on fast rows, the reciprocal r for row_quot.
// Fast rows take s from one Markstein step around k = RN(1 / 448) and r from the
// hardware reciprocal: on an MI355X, that s equals the IEEE quotient for every bf16
// amax in [2^-100, inf), and with that r the codes of row_quot equal those of the IEEE
// quotient x / s for every bf16 x with |x| <= amax (all pairs checked).  Other rows
// divide.
struct RowScale {
  float s, r;
  bool fast;
};
__device__ __forceinline__ RowScale row_scale(uint32_t amax_bits) {
  RowScale o;
  o.fast = row_quot_fast(amax_bits);
  if (o.fast) {
    constexpr float k = 1.0f / 448.0f;
    const float a = __uint_as_float(amax_bits);
    const float q0 = a * k;
    o.s = __builtin_fmaf(-__builtin_fmaf(q0, 448.0f, -a), k, q0);
    o.r = __builtin_amdgcn_rcpf(o.s);
  } else {
    o.s = scale_from_amax_bits(amax_bits);
    o.r = 0.0f;
  }
  return o;
}

// Two e4m3 codes (bytes 0,1 or 2,3 of w) -> two exact bf16 values.
template <bool kHigh>
__device__ __forceinline__ bf16x2_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHigh);
}

// Two e4m3 codes (bytes 0,1 or 2,3 of w) -> two exact float32 values.
template <bool kHigh>
__device__ __forceinline__ float2_t e4m3x2_to_f32x2(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, kHigh);
}

__device__ __forceinline__ float dot2_bf16(bf16x2_t a, bf16x2_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) {
  return __builtin_bit_cast(bf16x2_t, w);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return float_to_bf16_bits(lo) | (float_to_bf16_bits(hi) << 16);
}

// ---- cross-lane moves inside a 16-lane row (DPP) --------------------------------
// dpp_ctrl values of the gfx9 encoding.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i inside 8 (i ^ 7)
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i inside 16 (i ^ 15)

template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF,
                                                    0xF, false));
}

template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_mov_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kCtrl, 0xF, 0xF, false);
}

// Partner masks for lane bits 0..3 inside a row: bit b uses xor kXorOfBit[b].
// The pairing for bit b may also flip lower bits; the butterfly below only relies
// on it flipping bit b and leaving higher bits alone.
template <int kBit>
__device__ __forceinline__ float dpp_partner(float x) {
  if constexpr (kBit == 0) return dpp_mov<kDppXor1>(x);
  else if constexpr (kBit == 1) return dpp_mov<kDppXor2>(x);
  else if constexpr (kBit == 2) return dpp_mov<kDppHalfMirror>(x);
  else return dpp_mov<kDppMirror>(x);
}

// The values of lanes i and i ^ kSpan (kSpan 16 or 32), in some order, in every lane
// i: v_permlane16_swap / v_permlane32_swap of x with itself.  Whichever halves the
// instruction exchanges, one result holds x of lane i and the other x of its partner.
template <int kSpan>
__device__ __forceinline__ void lane_swap_pair(float x, float& a, float& b) {
  const uint32_t u = __float_as_uint(x);
  if constexpr (kSpan == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else {
    static_assert(kSpan == 32, "span");
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  }
}

// max(x of lane i, x of lane i ^ kSpan) / the sum of the two, in every lane
template <int kSpan = 32>
__device__ __forceinline__ float max_xor(float x) {
  float a, b;
  lane_swap_pair<kSpan>(x, a, b);
  return fmaxf(a, b);
}
template <int kSpan = 32>
__device__ __forceinline__ float sum_xor(float x) {
  float a, b;
  lane_swap_pair<kSpan>(x, a, b);
  return a + b;
}

// Maximum / sum over the 64 lanes, in every lane, all on the vector ALU (no LDS
// round trips): a butterfly over the four lane bits of a 16-lane row by DPP, then
// across rows by the two lane swaps.  Every lane of the wave must be active.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_partner<0>(x));
  x = fmaxf(x, dpp_partner<1>(x));
  x = fmaxf(x, dpp_partner<2>(x));
  x = fmaxf(x, dpp_partner<3>(x));
  float a, b;
  lane_swap_pair<16>(x, a, b);
  return max_xor<32>(fmaxf(a, b));
}

// Maximum over the 64 lanes of unsigned values (also the maximum of non-negative
// floats by their bits), in every lane.  Every lane of the wave must be active.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_mov_u<kDppXor1>(x));
  x = max(x, dpp_mov_u<kDppXor2>(x));
  x = max(x, dpp_mov_u<kDppHalfMirror>(x));
  x = max(x, dpp_mov_u<kDppMirror>(x));
  const auto r16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = max((uint32_t)r16[0], (uint32_t)r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max((uint32_t)r32[0], (uint32_t)r32[1]);
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_partner<0>(x);
  x += dpp_partner<1>(x);
  x += dpp_partner<2>(x);
  x += dpp_partner<3>(x);
  float a, b;
  lane_swap_pair<16>(x, a, b);
  return sum_xor<32>(a + b);
}

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Stores one (token, KV head) row of the cache: D bf16 values of K and of V, owned by
// D / 8 consecutive lanes (lane c of the group holds values 8c .. 8c + 7) that must be
// active together.  fp8: per-tensor scales k_scale / v_scale, or per-token-head scales
// amax / 448 computed here and stored in the scale pools; codes are RNE/saturating
// e4m3 of x / scale.  K goes token-major (tile, off, d), V dim-major (tile, d, off).
template <int D, bool kFp8, bool kPerTokenHead>
__device__ __forceinline__ void store_token_row(const uint16_t* k, const uint16_t* v, int c,
                                                int64_t tile, int off, uint8_t* k_pages,
                                                uint8_t* v_pages, float* k_scales,
                                                float* v_scales, float k_scale,
                                                float v_scale) {
  constexpr int kLanesPerRow = D / 8;
  const uint4 kw = *reinterpret_cast<const uint4*>(k + c * 8);
  const uint4 vw = *reinterpret_cast<const uint4*>(v + c * 8);
  const uint32_t kk[4] = {kw.x, kw.y, kw.z, kw.w};
  const uint32_t vv[4] = {vw.x, vw.y, vw.z, vw.w};
  if constexpr (!kFp8) {
    // bf16 cache (sliding-window layers kept unquantised): plain copy.
    uint16_t* kp = reinterpret_cast<uint16_t*>(k_pages);
    uint16_t* vp = reinterpret_cast<uint16_t*>(v_pages);
    *reinterpret_cast<uint4*>(kp + (tile * kPage + off) * D + c * 8) = kw;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      vp[(tile * D + c * 8 + 2 * i) * kPage + off] = (uint16_t)(vv[i] & 0xFFFFu);
      vp[(tile * D + c * 8 + 2 * i + 1) * kPage + off] = (uint16_t)(vv[i] >> 16);
    }
  } else {
    float kf[8], vf[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kf[2 * i] = bf16_bits_to_float(kk[i] & 0xFFFFu);
      kf[2 * i + 1] = bf16_bits_to_float(kk[i] >> 16);
      vf[2 * i] = bf16_bits_to_float(vv[i] & 0xFFFFu);
      vf[2 * i + 1] = bf16_bits_to_float(vv[i] >> 16);
    }
    float ks = k_scale, vs = v_scale;
    float kr = 0.0f, vr = 0.0f;     // per-token-head: 1 / scale for the fast quotient
    bool kfast = false, vfast = false;
    if constexpr (kPerTokenHead) {
      const uint32_t kv = row_amax_bf16_kv<kLanesPerRow>(kw, vw);
      const uint32_t ka = kv << 16, va = kv & 0xFFFF0000u;  // float32 magnitude bits
      const RowScale krs = row_scale(ka), vrs = row_scale(va);
      ks = krs.s;
      vs = vrs.s;
      kr = krs.r;
      vr = vrs.r;
      kfast = krs.fast;
      vfast = vrs.fast;
      if (c == 0) {
        k_scales[tile * kPage + off] = ks;
        v_scales[tile * kPage + off] = vs;
      }
    }
    *reinterpret_cast<uint2*>(k_pages + (tile * kPage + off) * D + c * 8) =
        make_uint2(e4m3_quantize4_row(kf, ks, kr, kfast), e4m3_quantize4_row(kf + 4, ks, kr, kfast));
    const uint32_t vlo = e4m3_quantize4_row(vf, vs, vr, vfast);
    const uint32_t vhi = e4m3_quantize4_row(vf + 4, vs, vr, vfast);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      v_pages[(tile * D + c * 8 + i) * kPage + off] = (uint8_t)((i < 4 ? vlo : vhi) >> (8 * (i % 4)));
  }
}

// Direct global -> LDS loads (each lane's 16 or 4 bytes land at lds_off + lane * size).
// Written as inline assembly on purpose: the compiler treats its own form of these
// loads as pending LDS writes and waits for all of them before any LDS read, which
// would drain the tile pipeline; here the waits are explicit (wait_vmcnt), and
// unknown vector memory operations can only make the compiler's own waits stricter.
__device__ __forceinline__ void lds_load16(const void* src, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(lds_off) : "memory", "m0");
}
// The same with a uniform 64-bit base in scalar registers and a 32-bit per-lane offset.
__device__ __forceinline__ void lds_load16s(const void* base, uint32_t voff, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(base), "s"(lds_off) : "memory", "m0");
}
__device__ __forceinline__ void lds_load4(const void* src, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(src), "s"(lds_off) : "memory", "m0");
}
template <typename T>
__device__ __forceinline__ uint32_t lds_offset(T* p) {  // p points into __shared__ memory
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8).  wait_vmcnt<N>: at most N vector memory operations outstanding, the other
// counters untouched.  barrier_lds: this wave's LDS operations done, then the
// workgroup barrier (unlike __syncthreads it does not wait for the direct-to-LDS
// loads still in flight).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

}  // namespace kvq
