// Device-side helpers shared by the HIP kernels of libtp (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tp {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// 16-byte chunk moved between HBM, registers and LDS.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// GELU, exact form: x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)).  The pages
// write the MLP as GELU(XA)B and name no approximation.
__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}

// Slope of the exact GELU for fp32 outputs: Phi(z) + z phi(z) with the
// device erff and expf.
__device__ __forceinline__ float gelu_grad_erf(float z) {
  return 0.5f * (1.0f + erff(z * 0.70710678118654752f)) + z * 0.39894228040143268f * expf(-0.5f * z * z);
}

// SiLU with beta = 1: g * sigmoid(g) = g / (1 + e^-g).
__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// GELU for bf16 outputs: the same exact (erf) form, GELU(z) = z Phi(z), with
// the Gaussian tail Q(x) = Phi(-x) = erfc(x / sqrt 2) / 2 (x >= 0) evaluated
// as an exponential of a polynomial:
//   Q(x) = 2^( -x^2 log2(e) / 2 + g(min(x, 5)) ),
// g a degree-6 least-squares fit of (ln Q(x) + x^2/2) log2(e) on [0, 5] (a
// smooth, slowly varying function: ln 1/2 at 0, about -ln(x sqrt(2 pi)) for
// large x).  Relative error of Q <= 1.6e-5 on [0, 5] in fp32, absolute error
// of GELU <= 2e-6 everywhere; past x = 5 (Q < 3e-7) the fit is held at 5.
// csrc/gelu_tail_fit.py fits the coefficients and checks these bounds.  Then
//   GELU(z) = max(z, 0) - |z| Q(|z|)
// (no cancellation of 1 + erf near -1): one exp2 and ten other operations,
// no reciprocal, no branch.
constexpr float kGeluNegHalfLog2e = (float)(-0.5 * 1.4426950408889634);
constexpr float kQc0 = -1.000011682510376f, kQc1 = -1.1509265899658203f, kQc2 = 0.2618351876735687f,
                kQc3 = -0.052690327167510986f, kQc4 = 0.007775241509079933f, kQc5 = -0.000713575107511133f,
                kQc6 = 2.9757440643152222e-05f;
constexpr float kQxMax = 5.0f;
// g(min(x, 5)) for x = |z|
__device__ __forceinline__ float gauss_tail_poly(float x) {
  const float u = fminf(x, kQxMax);
  return fmaf(fmaf(fmaf(fmaf(fmaf(fmaf(kQc6, u, kQc5), u, kQc4), u, kQc3), u, kQc2), u, kQc1), u, kQc0);
}
__device__ __forceinline__ float gelu_bf16out(float z) {
  const float q = __builtin_amdgcn_exp2f(fmaf(z * kGeluNegHalfLog2e, z, gauss_tail_poly(fabsf(z))));
  return fmaf(-fabsf(z), q, fmaxf(z, 0.0f));
}

// Slope of the exact GELU for bf16 outputs:
//   d/dz [z Phi(z)] = Phi(z) + z phi(z),  phi(z) = e^(-z^2/2) / sqrt(2 pi),
// with the tail Phi(-|z|) = Q(|z|) of gelu_bf16out (its fit and bounds) and
// phi from a second exp2 of the same exponent's quadratic part.
__device__ __forceinline__ float gelu_grad_bf16out(float z) {
  const float w = (z * kGeluNegHalfLog2e) * z;  // log2 e^(-z^2/2)
  const float q = __builtin_amdgcn_exp2f(w + gauss_tail_poly(fabsf(z)));  // Phi(-|z|)
  const float Phi = z >= 0.0f ? 1.0f - q : q;
  return fmaf(z * 0.39894228040143268f, __builtin_amdgcn_exp2f(w), Phi);
}

// SiLU for bf16 outputs: g / (1 + e^-g) with the hardware exponential and
// reciprocal (relative error ~1e-6, far below bf16 resolution).
__device__ __forceinline__ float silu_bf16out(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// Running (max, sum of exp(x - max)) pairs of the cross-entropy statistics.
// A pair with max = -inf holds nothing (sum 0); the side that holds the new
// max keeps its sum unscaled, so -inf never meets -inf in an exponential.
struct MaxSum {
  float m, s;
};

__device__ __forceinline__ MaxSum ms_merge(MaxSum a, MaxSum b) {
  const float mx = fmaxf(a.m, b.m);
  const float sa = a.m == mx ? a.s : a.s * __expf(a.m - mx);
  const float sb = b.m == mx ? b.s : b.s * __expf(b.m - mx);
  return {mx, sa + sb};
}

// Value of another lane of the same 16-lane DPP row (CTRL: a DPP control --
// quad_perm, row_half_mirror, row_mirror -- that stays inside the row).
template <int CTRL>
__device__ __forceinline__ float dpp_row(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Reduction over each 16-lane row: lanes xor 1, then xor 2 (quad_perm
// [1,0,3,2] and [2,3,0,1]) give every lane its quad's value; the half-row
// mirror (lane i <-> 7-i) joins the two quads of each half, the row mirror
// (i <-> 15-i) the two halves.  Every lane of the row ends with the result;
// the order of the operations is fixed.
template <class Op>
__device__ __forceinline__ float row16_reduce(float x, Op op) {
  x = op(x, dpp_row<0xB1>(x));
  x = op(x, dpp_row<0x4E>(x));
  x = op(x, dpp_row<0x141>(x));
  x = op(x, dpp_row<0x140>(x));
  return x;
}

// fp32 -> bf16, IEEE round-to-nearest-even (the compiler emits gfx950's
// v_cvt_pk_bf16_f32, which rounds to nearest even).
__device__ __forceinline__ bf16 to_bf16(float x) { return static_cast<bf16>(x); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Workgroups are handed to the 8 XCDs round-robin (workgroup w -> XCD w % 8).
// Renumber so that consecutive logical tile ids land on the same XCD and
// share its L2.  Works for any total (the last XCDs may get one tile fewer).
__device__ __forceinline__ int xcd_remap(int pid, int total) {
  constexpr int kXcd = 8;
  const int per = (total + kXcd - 1) / kXcd;
  int tall = total % kXcd;
  if (tall == 0) tall = kXcd;
  const int xcd = pid % kXcd;
  const int local = pid / kXcd;
  return xcd < tall ? xcd * per + local : tall * per + (xcd - tall) * (per - 1) + local;
}

}  // namespace tp
