// mix_ceiling.hip - the sustained matrix-core rate of gfx950 for the
// instruction mix of each attention kernel: libattn_ceiling.so.
//
// Not part of the attention path. A roofline fraction against the published
// bf16 peak (2.5 PFLOP/s: 256 CUs x 2.4 GHz x 4096 FLOP per clock) says how
// far a kernel is from the chip's nominal rate, not from what its own
// instruction mix can reach. This probe measures the latter: every wave
// issues 32x32x16 bf16 products back to back (four independent
// accumulators), and between them, per 8 products, the vector-ALU and LDS
// instructions that the kernel issues per 8 products (read from its
// instruction counters): exponentials (v_exp_f32), other vector instructions
// (fma, multiply, add, bf16 packs), 16-byte and 8-byte transposing LDS reads
// that feed later products' operands. No global memory traffic, no barrier,
// no dependency between the vector work and the products: an upper bound for
// a kernel with that mix. Operands are random bf16 values (random bits of
// sign and mantissa, exponents around 1); mix 0 uses constant operands, which
// run at a much higher rate: the matrix cores' power depends on the data.
//
// Launch: 256 workgroups of 8 waves (two per SIMD, every CU of the chip).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_ceiling.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlocks = 256, kThreads = 512;
constexpr int kLdsWords = 4096;  // u32x4 entries: 64 KB of LDS per workgroup
// Workspace: 16 u32x4 of operands per thread, then 4096 u32x4 of LDS contents per workgroup.
constexpr size_t kOperandWords = (size_t)kBlocks * kThreads * 16;
constexpr size_t kWords = kOperandWords + (size_t)kBlocks * kLdsWords;

// Random bf16 pairs from a counter-based hash (splitmix64 finaliser): sign and
// 7 mantissa bits random, exponent 126 or 127 (|x| in [0.5, 2)).
__global__ void fill_kernel(u32x4* __restrict__ w, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  u32x4 v;
  for (int j = 0; j < 4; ++j) {
    uint64_t z = (uint64_t)i * 4 + j + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    const uint32_t lo = (uint32_t)(z & 0x80FFu) | 0x3F00u;
    const uint32_t hi = (uint32_t)((z >> 32) & 0x80FFu) | 0x3F00u;
    v[j] = (lo & 0xFFFFu) | (hi << 16);
  }
  w[i] = v;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Transposing 8-byte LDS read (ds_read_b64_tr_b16) of 8-byte entry idx.
__device__ __forceinline__ u32x2 read_tr8(const u32x4* base, int idx) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(reinterpret_cast<const unsigned char*>(base) + 8 * idx));
  return __builtin_bit_cast(u32x2, v);
}

// Per 8 products (one loop iteration): EXP exponentials (v_exp_f32, input
// through the neg/abs modifiers), PACK bf16 packs (v_cvt_pk_bf16_f32),
// OTHER further vector instructions (fma, multiply and add in turn), R16
// 16-byte LDS reads and R8 8-byte transposing LDS reads (ds_read_b64_tr_b16,
// in pairs). The vector instructions are single-instruction volatile asm
// statements (arithmetic only; no memory access), so each iteration issues
// exactly these counts; the values they produce are irrelevant. Every result
// is used besides:
// exponential e writes X[e], which the other instructions read; other
// instruction k updates Y[k] once per iteration from the exponentials just
// computed (a loop-carried value summed at the end, the exponentials'
// inputs); pack p writes word p / 4 of operand
// A[4 + p % 4], which a product consumes; the 16-byte reads refill B[j] and
// the 8-byte pairs A[j] (j < 4) right after product j consumed it. All LDS
// addresses are fixed per lane. RANDOM = false: constant operands.
template <bool RANDOM, int EXP, int PACK, int OTHER, int R16, int R8>
__global__ __launch_bounds__(kThreads) void mix_kernel(const u32x4* __restrict__ w, float* __restrict__ out, int iters) {
  static_assert(EXP >= 0 && EXP <= 16 && PACK <= 16 && OTHER <= 40 && R16 <= 8 && R8 <= 8 && R8 % 2 == 0,
                "mix within the register plan");
  __shared__ u32x4 lds[kLdsWords];
  const int t = blockIdx.x * kThreads + threadIdx.x;
  const u32x4* lsrc = w + kOperandWords + (size_t)blockIdx.x * kLdsWords;
  for (int i = threadIdx.x; i < kLdsWords; i += kThreads) lds[i] = lsrc[i];
  __syncthreads();
  u32x4 A[8], B[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (RANDOM) {
      A[i] = w[(size_t)t * 16 + i];
      B[i] = w[(size_t)t * 16 + 8 + i];
    } else {
      bf16x8 ca, cb;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        ca[j] = (__bf16)(0.001f * (float)(threadIdx.x + j));
        cb[j] = (__bf16)(0.002f * (float)j);
      }
      A[i] = __builtin_bit_cast(u32x4, ca);
      B[i] = __builtin_bit_cast(u32x4, cb);
    }
  }
  f32x16 acc[4] = {};
  float X[16], Y[40];
#pragma unroll
  for (int i = 0; i < 16; ++i) X[i] = 0.25f + 0.001f * (float)((threadIdx.x + i) & 63);
#pragma unroll
  for (int i = 0; i < 40; ++i) Y[i] = 0.5f + 0.001f * (float)i;
  const int ro = (threadIdx.x >> 6) * 512 + (threadIdx.x & 63);  // this lane's entry in its wave's block of 512
  for (int it = 0; it < iters; ++it) {
    // Alternate halves of the LDS array (bit 11 of the entry index) so that the reads stay in the loop; entry
    // rb + 64 r (r < 8) stays inside the wave's block of 512, and so do the 8-byte entries 2 rb + 128 r (+ 64).
    const int rb = ro ^ ((it & 1) << 11);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      acc[r & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, A[r]),
                                                           __builtin_bit_cast(bf16x8, B[r]), acc[r & 3], 0, 0, 0);
      // LDS: refill the operands product r just consumed.
      if (r < R16) B[r] = lds[rb + 64 * r];
      if (r < R8 / 2) {
        const u32x2 lo = read_tr8(lds, 2 * rb + 128 * r);
        const u32x2 hi = read_tr8(lds, 2 * rb + 128 * r + 64);
        A[r] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
      // This product's share of the exponentials, other instructions and packs.
#pragma unroll
      for (int e = r * EXP / 8; e < (r + 1) * EXP / 8; ++e)
        asm volatile("v_exp_f32 %0, -|%1|" : "=v"(X[e]) : "v"(Y[e % 40]));
#pragma unroll
      for (int k = r * OTHER / 8; k < (r + 1) * OTHER / 8; ++k) {
        const int e = EXP > 0 ? k * EXP / OTHER : k;
        const float xa = X[e % 16], xb = X[(e + 1) % (EXP > 0 ? EXP : 16)];
        if (k % 3 == 0) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(Y[k]) : "v"(xa), "v"(xb));
        else if (k % 3 == 1) asm volatile("v_mul_f32 %0, %0, %1" : "+v"(Y[k]) : "v"(xa));
        else asm volatile("v_add_f32 %0, %0, %1" : "+v"(Y[k]) : "v"(xb));
      }
#pragma unroll
      for (int q = r * PACK / 8; q < (r + 1) * PACK / 8; ++q) {
        uint32_t w;
        asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(w) : "v"(Y[q % 40]), "v"(X[q % (EXP > 0 ? EXP : 16)]));
        A[4 + q % 4][(q / 4) % 4] = w;
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += acc[0][i] + acc[1][i] + acc[2][i] + acc[3][i] + X[i];
#pragma unroll
  for (int i = 0; i < 40; ++i) s += Y[i];
#pragma unroll
  for (int i = 0; i < 8; ++i) s += (float)(A[i][0] ^ B[i][1]);
  out[t] = s;
}

template <bool RANDOM, int EXP, int PACK, int OTHER, int R16, int R8>
hipError_t launch(const u32x4* w, float* out, int iters, hipStream_t s) {
  hipLaunchKernelGGL((mix_kernel<RANDOM, EXP, PACK, OTHER, R16, R8>), dim3(kBlocks), dim3(kThreads), 0, s, w, out,
                     iters);
  return hipGetLastError();
}

// Per 8 products: exponentials, packs, other vector instructions, 16-byte and 8-byte LDS reads. The
// exponential and LDS counts are the kernels' (SQ_INSTS_VALU_TRANS_F32, SQ_INSTS_LDS per product x 8); the
// other count is set so that the loop's vector instructions (with the 2 the loop itself needs) total the
// kernel's SQ_INSTS_VALU per product x 8, less the products: 36, 51, 54 and 30.
hipError_t launch_mix(int mix, const u32x4* w, float* out, int iters, hipStream_t s) {
  switch (mix) {
    case ATTN_MIX_CONSTANT: return launch<false, 0, 0, 0, 0, 0>(w, out, iters, s);
    case ATTN_MIX_RANDOM: return launch<true, 0, 0, 0, 0, 0>(w, out, iters, s);
    case ATTN_MIX_DKDV: return launch<true, 8, 8, 18, 8, 8>(w, out, iters, s);
    case ATTN_MIX_DQ: return launch<true, 11, 5, 22, 2, 4>(w, out, iters, s);
    case ATTN_MIX_FWD64: return launch<true, 16, 8, 28, 4, 8>(w, out, iters, s);
    case ATTN_MIX_FWD128: return launch<true, 8, 4, 14, 4, 8>(w, out, iters, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

extern "C" size_t attn_mix_ceiling_workspace_bytes(void) {
  return kWords * sizeof(u32x4) + (size_t)kBlocks * kThreads * sizeof(float);
}

extern "C" double attn_mix_ceiling_flop(int iters) {
  return (double)kBlocks * (kThreads / 64) * (double)iters * 8.0 * 32768.0;
}

extern "C" int attn_mix_ceiling(int mix, int iters, void* workspace, size_t workspace_bytes, float* ms, void* stream) {
  if (mix < ATTN_MIX_CONSTANT || mix > ATTN_MIX_FWD128 || iters < 1 || !workspace || !ms ||
      ((uintptr_t)workspace & 15) != 0)
    return -1;
  if (workspace_bytes < attn_mix_ceiling_workspace_bytes()) return -3;
  hipStream_t s = static_cast<hipStream_t>(stream);
  u32x4* w = static_cast<u32x4*>(workspace);
  float* out = reinterpret_cast<float*>(w + kWords);
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((kWords + 255) / 256)), dim3(256), 0, s, w, kWords);
  if (hipGetLastError() != hipSuccess) return -4;
  for (int i = 0; i < 3; ++i)
    if (launch_mix(mix, w, out, iters, s) != hipSuccess) return -4;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return -4;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return -4;
  }
  const int reps = 10;
  int rc = 0;
  if (hipEventRecord(e0, s) != hipSuccess) rc = -4;
  for (int i = 0; rc == 0 && i < reps; ++i)
    if (launch_mix(mix, w, out, iters, s) != hipSuccess) rc = -4;
  if (rc == 0 && hipEventRecord(e1, s) != hipSuccess) rc = -4;
  if (rc == 0 && hipEventSynchronize(e1) != hipSuccess) rc = -4;
  float t = 0.f;
  if (rc == 0 && hipEventElapsedTime(&t, e0, e1) != hipSuccess) rc = -4;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (rc == 0) *ms = t / reps;
  return rc;
}
