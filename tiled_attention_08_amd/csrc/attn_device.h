// attn_device.h - device-side building blocks shared by the attention kernels
// (gfx950 / CDNA4, wave64).
//
// Matrix-core conventions used throughout (v_mfma_f32_32x32x16_bf16, checked
// on the hardware with an in-bounds lane-layout probe; the _f16 form has the
// same layout, which the fp16 parity tests confirm):
//   A (32 x 16, M x K): lane l supplies A[l % 32][8 * (l / 32) + s], s = 0..7
//   B (16 x 32, K x N): lane l supplies B[8 * (l / 32) + s][l % 32]
//   D (32 x 32):        lane l holds D[8 * j + 4 * (l / 32) + i][l % 32] in acc[4 * j + i]
// The contraction index K may be permuted freely as long as A and B use the
// same permutation; the kernels use the one that makes an accumulator tile
// feed the next MFMA's B operand directly from registers: within a 16-wide
// k-chunk, half h = l / 32 holds k = 4h + {0..3} in slots 0..3 and
// k = 8 + 4h + {0..3} in slots 4..7.
//
// Transposing LDS read (ds_read_b64_tr_b16, also probed): within each group
// of 16 lanes, lane i receives element (i % 4) of the 8-byte rows addressed by
// lanes 4e + i / 4, for e = 0..3. If lane 4e + q of the group addresses
// row (r0 + e), columns (c0 + 4q .. c0 + 4q + 3) of a row-major bf16 tile,
// lane i ends up with column c0 + i of rows r0 .. r0 + 3: a transposed
// operand read straight from a row-major tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Compile-time boolean tag for code paths specialised on a flag.
template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

template <int V>
struct IntC {
  static constexpr int value = V;
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// lo.x + hi.x accumulated in fp32 (v_dot2_f32_bf16 against (1, 1)).
__device__ __forceinline__ float sum_bf16_pair(uint32_t pk, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), one, acc, false);
}

// Eight 16-bit elements from two 4-element halves.
__device__ __forceinline__ u32x4 cat(const u32x2& lo, const u32x2& hi) { return u32x4{lo[0], lo[1], hi[0], hi[1]}; }

// The 16-bit element types of storage and matrix-core operands. Fragments
// are carried as raw 32-bit words (a u32x4 holds 8 elements, a uint32_t a
// pair, low half first); each type supplies the 32x32x16 product with fp32
// accumulation, round-to-nearest-even packing of two floats, the fp32 sum of
// a packed pair (v_dot2 against (1, 1)) and the widening of each half.
struct Bf16 {
  __device__ static __forceinline__ f32x16 mfma(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ uint32_t pack(float lo, float hi) { return pack_bf16(lo, hi); }
  __device__ static __forceinline__ float sum_pair(uint32_t pk, float acc) { return sum_bf16_pair(pk, acc); }
  __device__ static __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
  __device__ static __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
};

struct F16 {
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  __device__ static __forceinline__ f32x16 mfma(const u32x4& a, const u32x4& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
  // v_cvt_pk_f16_f32 (round to nearest even).
  __device__ static __forceinline__ uint32_t pack(float lo, float hi) {
    f16x2 v;
    v[0] = (_Float16)lo;
    v[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ static __forceinline__ float sum_pair(uint32_t pk, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk), one, acc, false);
  }
  __device__ static __forceinline__ float lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)w); }
  __device__ static __forceinline__ float hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
};

// NaN-propagating maxima (v_maximum3_f32 on gfx950). Unlike fmaxf they need
// no canonicalising copy of each operand.
__device__ __forceinline__ float fmax2(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float fmax3(float a, float b, float c) {
  return __builtin_elementwise_maximum(a, __builtin_elementwise_maximum(b, c));
}

// Maximum of N values as a tree of three-operand maxima over distinct operands
// (about (N - 1) / 2 instructions). Written as a running chain
// max(m, max(a, b)), the compiler re-associates it into three instructions
// per four values.
template <int N>
__device__ __forceinline__ float max_tree(const float* x) {
  if constexpr (N == 1) {
    return x[0];
  } else if constexpr (N == 2) {
    return fmax2(x[0], x[1]);
  } else if constexpr (N == 3) {
    return fmax3(x[0], x[1], x[2]);
  } else {
    constexpr int G = (N + 2) / 3;
    float y[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
      y[g] = 3 * g + 2 < N ? fmax3(x[3 * g], x[3 * g + 1], x[3 * g + 2])
                           : (3 * g + 1 < N ? fmax2(x[3 * g], x[3 * g + 1]) : x[3 * g]);
    return max_tree<G>(y);
  }
}

// max / sum of x over lanes l and l ^ 32.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmax2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS tile swizzle. Tiles are row-major 16-bit elements in 16-byte chunks (8
// elements); chunk c of row r is stored at chunk position c ^ swz(r). Two read
// patterns must be free of bank conflicts (64 banks of 4 bytes, so a 256-byte
// window of LDS covers every bank once):
//   plain 16-byte reads: gfx950 serves a ds_read_b128 in 16-lane quarters,
//     and the 16 lanes of an operand read (16 consecutive rows, the same
//     logical chunk) must hit 16 distinct 16-byte bank groups;
//   transposing 8-byte reads: a 32-lane half of a ds_read_b64_tr_b16 reads 4
//     consecutive rows (the first a multiple of 4) x 4 consecutive chunks
//     (the first a multiple of 4), 8 bytes per lane, and its 16 (row, chunk)
//     pairs must hit 16 distinct bank groups.
// Row sizes and swizzles:
//   128-byte rows (two rows per window, an odd row in the other half):
//     swz(r) = bit-reverse of the 3 bits (r >> 1) & 7. The 8 rows of each
//     parity among 16 consecutive rows take 8 different positions, and rows
//     r and r + 2 (r a multiple of 4, same half window) differ in bit 2, so
//     their 4-chunk groups land in opposite halves of the row.
//   256-byte rows (one row per window): swz(r) = bit-reverse of the 4 bits
//     r & 15: a bijection over 16 consecutive rows, and rows r .. r + 3 (r a
//     multiple of 4) differ in bits 2 and 3, so their 4-chunk groups take
//     all 16 positions.
//   64-byte rows (four rows per window) and 192-byte rows (rows start at
//     window offsets 0, 192, 128, 64 in turn): swz(r) = (r >> 2) & 3, which
//     spreads each group of four rows with the same window offset over four
//     slots (and keeps the chunk index below 12 for 192-byte rows).
// (The plain XOR swizzles (r >> 1) & 7 and r & 15 are conflict-free for the
// plain reads but put two or four lanes on one bank in the transposing reads.)
template <int ROWB>
__device__ __forceinline__ int swz(int row) {
  static_assert(ROWB == 64 || ROWB == 128 || ROWB == 192 || ROWB == 256, "tiles have 64 to 256-byte rows");
  if constexpr (ROWB == 128) return (int)(__builtin_bitreverse32((uint32_t)row >> 1) >> 29);
  if constexpr (ROWB == 256) return (int)(__builtin_bitreverse32((uint32_t)row) >> 28);
  return (row >> 2) & 3;
}

// Byte offset of element (row, col) in a swizzled tile with ROWB bytes per row.
template <int ROWB>
__device__ __forceinline__ int tile_off(int row, int col) {
  const int chunk = col >> 3;
  return row * ROWB + ((chunk ^ swz<ROWB>(row)) << 4) + ((col & 7) << 1);
}

__device__ __forceinline__ u32x4 lds_read_b128(const unsigned char* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}

__device__ __forceinline__ u32x2 lds_read_tr16_b64(const unsigned char* base, int off) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off));
  return __builtin_bit_cast(u32x2, v);
}

// Asynchronous 16-byte copy global -> LDS (global_load_lds_dwordx4): lane l of
// the wave writes the 16 bytes at `src` to LDS address lds_base + 16 * l.
// `lds_base` must be wave-uniform. Completion is tracked by vmcnt.
__device__ __forceinline__ void dma16(const void* src, unsigned char* lds_base) {
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_base, 16, 0, 0);
}

// Same with 4 bytes per lane (global_load_lds_dword): lane l writes lds_base + 4 * l.
__device__ __forceinline__ void dma4(const void* src, unsigned char* lds_base) {
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_global_load_lds(src, (lds_void*)lds_base, 4, 0, 0);
}

// The same copies through a buffer resource (buffer_load_dword{,x4} ... lds):
// lane l writes lds_base + size * l with the bytes at byte offset `off` of the
// resource. The attention kernels use these: the compiler counts a
// global_load_lds as both a vector-memory and an LDS access and, while one is
// in flight, makes every LDS read wait for all LDS reads issued (lgkmcnt(0)),
// which defeats reading operands ahead; buffer copies count as vector memory
// only. A resource covers one head of one tensor (offsets below 2^31, which
// the host-side index checks guarantee); word 3 is the gfx9 raw-buffer format.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ void dma16(Rsrc r, uint32_t off, unsigned char* lds_base) {
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void dma4(Rsrc r, uint32_t off, unsigned char* lds_base) {
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 4, off, 0, 0, 0);
}

// Wait until every outstanding global load of this wave (including LDS DMA) has landed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt encoding (gfx9): wait until at most N vector-memory operations of
// this wave are outstanding; LGKM and export counters are left alone.
template <int N>
__device__ __forceinline__ void wait_vmem_below() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Calls f(IntC<I>{}) for I = B .. E-1 in order (compile-time indices).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(IntC<B>{});
    static_for<B + 1, E>(f);
  }
}

// Work-item index for a 1-D grid, grouping consecutive work items on one XCD.
// Workgroups are handed to the 8 XCDs round-robin by launch index; this
// bijection gives XCD x a contiguous block of work items (the same heads, so
// the same K/V stay in that XCD's L2).
__device__ __forceinline__ int xcd_remap(int id, int total) {
  const int x = id & 7, slot = id >> 3, per = total >> 3, rem = total & 7;
  return x * per + (x < rem ? x : rem) + slot;
}

// Element strides of a group of [B, H, N, d] tensors: batch, head and row
// (token); the d elements of a row are contiguous. Contiguous [B,H,N,d] is
// {H N d, N d, d}; token-major [B,N,H,d] is {N H d, d, H d}; Q, K and V
// packed in one [B,N,3,H,d] buffer use {3 N H d, d, 3 H d} from their own
// base pointers.
struct Strides {
  long long b, h;
  int n;
};

// Offset of head (b, h) = (bh / H, bh % H).
__device__ __forceinline__ size_t head_off(const Strides& s, int bh, int H) {
  const int b = bh / H;
  return (size_t)b * (size_t)s.b + (size_t)(bh - b * H) * (size_t)s.h;
}

// (head, block) of work item `work` (after xcd_remap) for a grid of total =
// heads * n_blk items. Plain order: head-major, block ascending. With
// `causal`, blocks carry unequal work (the block with the most is n_blk - 1
// when heavy_last, else 0) and are handed out heaviest first: when each XCD's
// range holds whole heads, every group of ATTN_CAUSAL_GROUP heads in it is
// ordered by block (heaviest first), then head, so every XCD keeps its own
// heads (and their K/V in its L2) while the long blocks of a group start
// before any short one; otherwise blocks are reversed within each head.
// Heads per heaviest-first group: the XCD's range is worked through group by
// group, heaviest blocks first inside each group, so that the K/V (or Q/dO) of
// only a few heads compete for its L2 at a time. Measured on the causal
// B=8, H=16, N=4096 step: 8 heads 1347 us, all 16 at once 1379 us, 4 heads
// 1365 us, 2 heads 1451 us.
#ifndef ATTN_CAUSAL_GROUP
#define ATTN_CAUSAL_GROUP 8
#endif
__device__ __forceinline__ void work_order(int work, int total, int n_blk, bool causal, bool heavy_last, int& bh,
                                           int& blk) {
  bh = work / n_blk;
  blk = work - bh * n_blk;
  if (!causal) return;
  const int per = total >> 3;
  if ((total & 7) == 0 && per % n_blk == 0) {
    const int hpx = per / n_blk, x = work / per, r = work - x * per;
    const int G = (ATTN_CAUSAL_GROUP > 0 && hpx % ATTN_CAUSAL_GROUP == 0) ? ATTN_CAUSAL_GROUP : hpx;
    const int grp = r / (G * n_blk), rg = r - grp * G * n_blk, rank = rg / G;
    bh = x * hpx + grp * G + (rg - rank * G);
    blk = rank;
  }
  if (heavy_last) blk = n_blk - 1 - blk;
}

}  // namespace attn
