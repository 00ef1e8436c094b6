// Device-side pieces shared by the GEMM kernels: the int4 / int8 dequant
// of packed weight words into fp16 MFMA operands, and the kernel arguments.
#pragma once
#include "common.h"

namespace dfl {

// --------------------------------------------------------------- dequant
__device__ __forceinline__ half2v h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }

// (a & m) | c in one VALU op (the compiler splits it into two)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(c));
  return r;
}

// 8 int4 codes (one dword, offset binary, nibble slots as packed) -> 8 halves
// 0x6400 | u is the fp16 value 1024 + u; (0x6400 | 16u) scaled by 1/16 is 64 + u.
// mlo = 0x000F000F, mhi = 0x00F000F0, magic = 0x64006400 (register operands).
__device__ __forceinline__ half8 deq_w4(uint32_t w, uint32_t mlo, uint32_t mhi, uint32_t magic) {
  const half2v c0 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const half2v s16 = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2v c1 = {(_Float16)-72.0f, (_Float16)-72.0f};
  const uint32_t w2 = w >> 8;
  half2v a = h2(and_or(w, mlo, magic)) + c0;
  half2v b = h2(and_or(w, mhi, magic)) * s16 + c1;
  half2v c = h2(and_or(w2, mlo, magic)) + c0;
  half2v d = h2(and_or(w2, mhi, magic)) * s16 + c1;
  half8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}

// 8 int4 codes (one dword, offset binary, nibble slots as packed) -> the 8
// fp16 subnormals c * 2^-24 in deq_w4's order: with mlo = 0x000F000F each AND
// leaves one code in the low bits of each half
__device__ __forceinline__ half8 deq_w4_sub(uint32_t w, uint32_t mlo) {
  const uint32_t a = w & mlo, b = (w >> 4) & mlo, c = (w >> 8) & mlo, d = (w >> 12) & mlo;
  return __builtin_bit_cast(half8, uint4{a, b, c, d});
}

// 8 int8 codes (two dwords, bytes in column order, offset binary) -> 8 halves:
// byte pairs are spread to the low bytes of two fp16 lanes over the magic 0x64.
__device__ __forceinline__ half8 deq_w8(uint32_t lo, uint32_t hi, uint32_t magic) {
  const half2v c = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  half2v a = h2(__builtin_amdgcn_perm(magic, lo, 0x05010500u)) + c;
  half2v b = h2(__builtin_amdgcn_perm(magic, lo, 0x05030502u)) + c;
  half2v d = h2(__builtin_amdgcn_perm(magic, hi, 0x05010500u)) + c;
  half2v e = h2(__builtin_amdgcn_perm(magic, hi, 0x05030502u)) + c;
  half8 r = {a[0], a[1], b[0], b[1], d[0], d[1], e[0], e[1]};
  return r;
}

// ------------------------------------------------------------ arguments
struct GemmArgs {
  const uint8_t* w; const uint16_t* s; const uint16_t* x;
  int n, k, ktiles, ntile16, m, splits, align;
  int epi;
  float* part;                               // EPI_PARTIAL: [splits][m][n] fp32
  void* out; int otype;                      // EPI_SILU: tiled [m][n/2] (K = n/2)
  float* logits; int ldl; int row0;          // EPI_ARGMAX
  float* am_val; int* am_idx;                // EPI_ARGMAX: one (value, index) per work-group and token
  int32_t* status;                           // EPI_SILU: range flag of fp16 outputs (or null)
  // dequant bit masks, passed as arguments so that they live in registers
  // (gfx9 VOP3 encodings take no literal constants)
  uint32_t mlo, mhi, magic;
};

// the dense prompt-chunk GEMM (gemm_dense.hip)
hipError_t launch_gemm_dense(const GemmCall& c, const Workspace& w, hipStream_t s, int* splits);

}  // namespace dfl
