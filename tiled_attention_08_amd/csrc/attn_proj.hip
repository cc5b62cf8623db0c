// attn_proj.hip - the query/key/value projection that feeds attention, and its
// backward, on the gfx950 matrix cores.
//
// Article "Selbstaufmerksamkeit, CUDA-Kernel und FlashAttention" (German
// edition of the self-attention / Triton / FlashAttention article,
// itimpress.au, 2026-11-15), §1 first bullet: the token matrix X (one row per
// patch, D columns) is multiplied by three learned D x d_k matrices per head,
// Q = X W_Q, K = X W_K, V = X W_V. With the weights of all heads side by side,
// w[D, 3, H, d_k], this is one product per batch of tokens:
//   forward  qkv[BN, 3Hd] = x[BN, D] w[D, 3Hd]      (qkv is [B, N, 3, H, d_k],
//            the packed layout the attention entry points read);
//   dx       dx[BN, D]    = dqkv[BN, 3Hd] w^T;
//   dw       dw[D, 3Hd]   = x^T dqkv, summed over all B N tokens.
//
// Every product is C = A B (A: M x K, B: K x N, fp32 accumulation, C rounded
// once to the 16-bit storage type). An operand is "k-contiguous" when its
// contraction index runs along memory rows (A row-major, or B stored as B^T
// row-major). Such an operand is staged as [rows][64 k] tiles and read with
// plain 16-byte LDS reads. Otherwise it is staged as [64 k][cols] tiles and
// read with the transposing LDS read, so no operand is ever transposed in
// memory:
//   forward: A = x (k-contiguous), B = w (not);
//   dx:      A = dqkv (k-contiguous), B = w^T, i.e. the rows of w (k-contiguous);
//   dw:      A = x^T (not), B = dqkv (not).
// Waves compute blocks of C^T = B^T A^T with 32x32x16 MFMAs: a lane then holds
// one row of C and stores four consecutive columns of it at a time.
// Two kernels:
//   gemm256_kernel - 256 x 256 tiles, 8 waves, for products with at least 256
//     rows and columns; a product with few tiles splits its contraction over
//     several workgroups, which write float32 partial slices to the caller's
//     workspace for reduce_splits_kernel to add in a fixed order;
//   gemm_kernel - 128 x 128 or 64 x 64 tiles, 4 waves, for smaller products;
//     the 64 x 64 form splits the contraction over its 4 waves and adds their
//     partial sums through LDS.
#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {

namespace {

template <int WM, int WN, int WK>
struct GemmShape {
  static_assert(WM * WN * WK == 4, "four waves per workgroup");
  static constexpr int BM = 64 * WM, BN = 64 * WN;  // output tile (rows of C x columns of C)
  static constexpr int ASZ = BM * 64 * 2;             // one 64-deep A sub-tile, bytes
  static constexpr int BSZ = 64 * BN * 2;             // one 64-deep B sub-tile, bytes
  static constexpr int STEPB = WK * (ASZ + BSZ);      // one contraction step (64 WK deep)
  static constexpr int RED = (WK - 1) * WM * WN * 64 * 64 * 4;  // partial sums of waves wk > 0
  static constexpr int LDSB = 2 * STEPB > RED ? 2 * STEPB : RED;
};

// DMA one operand sub-tile into LDS. The tile has `rows` rows of ROWB bytes;
// the 256 threads fill its 16-byte slots in order, and the lane writing slot
// (row, s) fetches logical chunk s ^ swz(row) (the layout tile_off() addresses).
// Row r of the tile is global row min(r0 + r, rmax) of `src` (leading
// dimension ld elements); chunk c starts at global column min(c0 + 8 c, cmax).
// Clamped rows and columns re-read valid data; the products mask every use.
template <int ROWB, int ROWS>
__device__ __forceinline__ void dma_tile(const uint16_t* __restrict__ src, size_t ld, int r0, int rmax, int c0,
                                         int cmax, unsigned char* dst, int tid) {
  constexpr int CPR = ROWB / 16;             // 16-byte chunks per row
  constexpr int ITERS = ROWS * CPR / 256;    // slots per thread
  static_assert(ITERS >= 1 && ROWS * CPR % 256 == 0, "whole 256-slot passes");
  const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int slot0 = it * 256 + wave * 64;
    const int p = slot0 + lane;
    const int row = p / CPR, chunk = (p - row * CPR) ^ swz<ROWB>(row);
    const int gr = min(r0 + row, rmax);
    const int gc = min(c0 + chunk * 8, cmax);
    dma16(src + (size_t)gr * ld + gc, dst + slot0 * 16);
  }
}

// Zero the 16-bit elements of an 8-element fragment whose contraction index
// is past the end: slot s is kept iff s < kv.
__device__ __forceinline__ u32x4 mask_k(u32x4 f, int kv) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t keep = (2 * w < kv ? 0x0000ffffu : 0u) | (2 * w + 1 < kv ? 0xffff0000u : 0u);
    f[w] &= keep;
  }
  return f;
}

// C[M, N] = A[M, K] B[K, N].
//   AK: A element (m, k) at A[m lda + k], else at A[k lda + m];
//   BK: B element (k, n) at B[n ldb + k], else at B[k ldb + n].
// Requirements (checked by the caller): 16-byte aligned bases; lda, ldb, ldc
// multiples of 8; N a multiple of 4; for a k-contiguous operand K >= 8 and
// K a multiple of 8; for the others the non-contraction extent >= 8 and a
// multiple of 8.
template <class E, bool AK, bool BK, int WM, int WN, int WK>
__global__ __launch_bounds__(256, 2) void gemm_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ Bm,
                                                      uint16_t* __restrict__ C, int M, int N, int K, int lda, int ldb,
                                                      int ldc, int tiles_n, int total) {
  using S = GemmShape<WM, WN, WK>;
  constexpr int BM = S::BM, BN = S::BN;
  constexpr int AROWB = AK ? 128 : 2 * BM, BROWB = BK ? 128 : 2 * BN;
  __shared__ __attribute__((aligned(16))) unsigned char smem[S::LDSB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31, i16 = lane & 15, grp = (lane >> 4) & 1;
  const int wk = wave / (WM * WN), wr = wave - wk * (WM * WN), wm = wr / WN, wn = wr - wm * WN;
  const int work = xcd_remap(blockIdx.x, total);
  const int tm = work / tiles_n, tn = work - tm * tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  constexpr int KSTEP = 64 * WK;
  const int nsteps = (K + KSTEP - 1) / KSTEP;

  auto dma_step = [&](int s, int buf) {
    unsigned char* base = smem + buf * S::STEPB;
#pragma unroll
    for (int kw = 0; kw < WK; ++kw) {
      const int k0 = s * KSTEP + kw * 64;
      unsigned char* As = base + kw * (S::ASZ + S::BSZ);
      unsigned char* Bs = As + S::ASZ;
      if (AK)
        dma_tile<128, BM>(A, lda, m0, M - 1, k0, K - 8, As, tid);
      else
        dma_tile<2 * BM, 64>(A, lda, k0, K - 1, m0, M - 8, As, tid);
      if (BK)
        dma_tile<128, BN>(Bm, ldb, n0, N - 1, k0, K - 8, Bs, tid);
      else
        dma_tile<2 * BN, 64>(Bm, ldb, k0, K - 1, n0, N - 8, Bs, tid);
    }
  };

  f32x16 acc[2][2];  // [n block][m block] of C^T
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) acc[nb][mb] = f32x16{};

  // Fragment of the 32 rows r0 + l32 of a [rows][64 k] tile at contraction
  // offset kk * 16 + 8 h (plain read), or of the 32 columns c0 + l32 of a
  // [64 k][cols] tile (two transposing reads of 4 rows each).
  auto frag = [&](const unsigned char* T, auto kcontig, auto rowb, int rc0, int kk) -> u32x4 {
    constexpr int RB = decltype(rowb)::value;
    if constexpr (decltype(kcontig)::value) {
      return lds_read_b128(T, tile_off<RB>(rc0 + l32, kk * 16 + 8 * h));
    } else {
      const int col = rc0 + grp * 16 + 4 * (i16 & 3);
      const int row = kk * 16 + 8 * h + (i16 >> 2);
      return cat(lds_read_tr16_b64(T, tile_off<RB>(row, col)), lds_read_tr16_b64(T, tile_off<RB>(row + 4, col)));
    }
  };

  auto compute = [&](int s, int buf, auto masked) {
    const unsigned char* As = smem + buf * S::STEPB + wk * (S::ASZ + S::BSZ);
    const unsigned char* Bs = As + S::ASZ;
    const int kbase = s * KSTEP + wk * 64;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 af[2], bf[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) af[nb] = frag(Bs, BoolC<BK>{}, IntC<BROWB>{}, wn * 64 + nb * 32, kk);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) bf[mb] = frag(As, BoolC<AK>{}, IntC<AROWB>{}, wm * 64 + mb * 32, kk);
      if constexpr (decltype(masked)::value) {
        const int kv = K - (kbase + kk * 16 + 8 * h);
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          af[x] = mask_k(af[x], kv);
          bf[x] = mask_k(bf[x], kv);
        }
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) acc[nb][mb] = E::mfma(af[nb], bf[mb], acc[nb][mb]);
    }
  };

  dma_step(0, 0);
  wait_vmem();
  __syncthreads();
  // Steps before the last read only indices below K; the last one may run past it.
  int s = 0;
  for (; s + 1 < nsteps; ++s) {
    const int buf = s & 1;
    dma_step(s + 1, buf ^ 1);
    compute(s, buf, BoolC<false>{});
    wait_vmem();
    __syncthreads();
  }
  if ((s + 1) * KSTEP <= K)
    compute(s, s & 1, BoolC<false>{});
  else
    compute(s, s & 1, BoolC<true>{});

  if constexpr (WK > 1) {
    // Waves wk > 0 leave their partial sums in LDS ([wave][register][lane],
    // 16 bytes per lane per store); waves wk == 0 add them up.
    __syncthreads();
    float4* red = reinterpret_cast<float4*>(smem);
    if (wk > 0) {
      const int slot = (wk - 1) * (WM * WN) + wr;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x16& a = acc[nb][mb];
            red[((slot * 16) + (nb * 2 + mb) * 4 + r4) * 64 + lane] =
                make_float4(a[4 * r4], a[4 * r4 + 1], a[4 * r4 + 2], a[4 * r4 + 3]);
          }
    }
    __syncthreads();
    if (wk > 0) return;
#pragma unroll
    for (int o = 1; o < WK; ++o) {
      const int slot = (o - 1) * (WM * WN) + wr;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const float4 v = red[((slot * 16) + (nb * 2 + mb) * 4 + r4) * 64 + lane];
            acc[nb][mb][4 * r4] += v.x;
            acc[nb][mb][4 * r4 + 1] += v.y;
            acc[nb][mb][4 * r4 + 2] += v.z;
            acc[nb][mb][4 * r4 + 3] += v.w;
          }
    }
  }

  // acc[nb][mb][4 j + i] = C[m][n] with m = m0 + wm 64 + mb 32 + l32 and
  // n = n0 + wn 64 + nb 32 + 8 j + 4 h + i: four consecutive columns per store.
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int m = m0 + wm * 64 + mb * 32 + l32;
    if (m >= M) continue;
    uint16_t* crow = C + (size_t)m * ldc;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 64 + nb * 32 + 8 * j + 4 * h;
        if (n < N) {
          const f32x16& a = acc[nb][mb];
          const u32x2 v = {E::pack(a[4 * j], a[4 * j + 1]), E::pack(a[4 * j + 2], a[4 * j + 3])};
          *reinterpret_cast<u32x2*>(crow + n) = v;
        }
      }
  }
}

// ---------------------------------------------------------------- large tiles
// 256 x 256 output tiles, 8 waves (2 along M x 4 along N, each 128 x 64 of C),
// two 64-deep LDS stages (64 KB each). One contraction step is 32 MFMAs per
// wave, about 2000 clocks per SIMD with its two waves, which covers the
// latency of the next stage's loads. Optionally the contraction is split S
// ways over S workgroups per tile (for products with few output tiles): split
// s then writes its float32 partial C to slice s of the workspace, and a
// second kernel adds the S slices in split order and rounds once. Results do
// not depend on the order in which workgroups run.
#ifndef PROJ_G2_REMAT
#define PROJ_G2_REMAT 1
#endif
#ifndef PROJ_G2_SCHED
#define PROJ_G2_SCHED 1
#endif
#ifndef PROJ_G2_SPLIT
#define PROJ_G2_SPLIT 1
#endif
constexpr int G2_THREADS = 512;
constexpr int G2_TILE = 256;
constexpr int G2_STAGEB = 2 * G2_TILE * 64 * 2;  // A and B sub-tiles of one stage

// Byte offset of a copy lane that must read zeros: at or past the resource's
// record count (0x7fffffff), so the buffer load returns zeros and touches no
// memory; LDS then holds exact zeros there and the products need no masking.
constexpr uint32_t G2_ZERO_OFF = 0x80000000u;

// Largest leading dimension (elements) for which every copy offset of a stage,
// taken from the stage's origin, stays below 2^31 bytes: at most 255 rows of
// ld elements plus one row.
constexpr long G2_MAX_LD = ((1L << 30) - 256) / G2_TILE;

// As dma_tile, for 512 threads, through a buffer resource based at the
// operand element (ro, co) (row ro, column co of its memory layout); lanes
// whose global row is at or past rzero, or whose chunk starts at or past
// column czero, read zeros. The clamped rows and columns are >= (ro, co).
// Buffer copies count as vector-memory accesses only, so the compiler lets
// LDS reads of the other stage run while this copy is in flight.
template <int ROWB, int ROWS>
__device__ __forceinline__ void dma_tile512(Rsrc rs, int ld, int ro, int co, int r0, int rmax, int rzero, int c0,
                                            int cmax, int czero, unsigned char* dst, int tid) {
  constexpr int CPR = ROWB / 16;
  constexpr int ITERS = ROWS * CPR / G2_THREADS;
  static_assert(ITERS >= 1 && ROWS * CPR % G2_THREADS == 0, "whole 512-slot passes");
  const int wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int slot0 = it * G2_THREADS + wave * 64;
    const int p = slot0 + lane;
    const int row = p / CPR, chunk = (p - row * CPR) ^ swz<ROWB>(row);
    const int r = r0 + row, c = c0 + chunk * 8;
    const uint32_t off = (r >= rzero || c >= czero)
                             ? G2_ZERO_OFF
                             : 2u * ((uint32_t)(min(r, rmax) - ro) * (uint32_t)ld + (uint32_t)(min(c, cmax) - co));
    dma16(rs, off, dst + slot0 * 16);
  }
}

// One 256-wide operand sub-tile of a stage (A: rows of C; B: columns of C),
// contraction indices k0 .. k0 + 63, zero from kend on.
// k-contiguous: [256][64 k], 128-byte rows. Otherwise two [64 k][128] halves
// with 256-byte rows (half h holds columns 128 h .. 128 h + 127).
// xlim: rows (k-contiguous) or columns (otherwise) of the operand in memory.
template <bool KC>
__device__ __forceinline__ void dma_operand(const uint16_t* __restrict__ src, int ld, int x0, int xlim, int k0,
                                            int kend, unsigned char* dst, int tid) {
  if constexpr (KC) {
    const Rsrc rs = make_rsrc(src + (size_t)x0 * ld + k0);
    dma_tile512<128, G2_TILE>(rs, ld, x0, k0, x0, xlim - 1, INT32_MAX, k0, kend - 8, kend, dst, tid);
  } else {
    const Rsrc rs = make_rsrc(src + (size_t)k0 * ld + x0);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      dma_tile512<256, 64>(rs, ld, k0, x0, k0, kend - 1, kend, x0 + 128 * hf, xlim - 8, INT32_MAX,
                           dst + hf * (64 * 256), tid);
  }
}

// Fragment of the 32 rows / columns c0 + l32 of a 256-wide sub-tile at
// contraction offset kk * 16 + 8 h (the slot order of both MFMA operands).
template <bool KC>
__device__ __forceinline__ u32x4 frag256(const unsigned char* T, int c0, int kk, int lane) {
  const int h = lane >> 5, l32 = lane & 31;
  if constexpr (KC) {
    return lds_read_b128(T, tile_off<128>(c0 + l32, kk * 16 + 8 * h));
  } else {
    const int i16 = lane & 15, grp = (lane >> 4) & 1;
    const unsigned char* half = T + (c0 >> 7) * (64 * 256);
    const int col = (c0 & 127) + grp * 16 + 4 * (i16 & 3);
    const int row = kk * 16 + 8 * h + (i16 >> 2);
    return cat(lds_read_tr16_b64(half, tile_off<256>(row, col)), lds_read_tr16_b64(half, tile_off<256>(row + 4, col)));
  }
}

// C[M, N] = A[M, K] B[K, N] with the operand conventions of gemm_kernel.
// Grid: tiles * S workgroups, split-major. Split s covers contraction
// indices [s kchunk, min(K, (s + 1) kchunk)); kchunk is a multiple of 64.
// S == 1: C is stored (rounded). S > 1: the float32 sums go to
// part + s M N, row-major [M][N], for reduce_splits_kernel.
template <class E, bool AK, bool BK>
__global__ __launch_bounds__(G2_THREADS) void gemm256_kernel(const uint16_t* __restrict__ A,
                                                             const uint16_t* __restrict__ Bm, uint16_t* __restrict__ C,
                                                             int M, int N, int K, int lda, int ldb, int ldc,
                                                             int tiles_n, int tiles, int S, int kchunk,
                                                             float* __restrict__ part) {
#if PROJ_G2_SPLIT
  // One LDS array per stage, selected at compile time: the compiler then
  // tells the copy into one stage from the reads of the other, and lets the
  // next stage's copy run during this stage's products (with one array and a
  // runtime stage index it waited for every copy before the first read).
  __shared__ __attribute__((aligned(16))) unsigned char smem0[G2_STAGEB];
  __shared__ __attribute__((aligned(16))) unsigned char smem1[G2_STAGEB];
#else
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * G2_STAGEB];
#endif

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int wm = wave >> 2, wn = wave & 3;  // this wave: rows wm 128 .. +127, columns wn 64 .. +63 of the tile
  const int work = xcd_remap(blockIdx.x, tiles * S);
  const int s = work / tiles, t = work - s * tiles;
  const int tm = t / tiles_n, tn = t - tm * tiles_n;
  const int m0 = tm * G2_TILE, n0 = tn * G2_TILE;
  const int kbeg = s * kchunk, kend = min(K, kbeg + kchunk);
  const int nsteps = (kend - kbeg + 63) / 64;

#if PROJ_G2_SPLIT
  auto stage = [&](auto b_) __attribute__((always_inline)) -> unsigned char* {
    if constexpr (decltype(b_)::value == 0) return smem0;
    else return smem1;
  };
#else
  auto stage = [&](auto b_) __attribute__((always_inline)) -> unsigned char* {
    return smem + decltype(b_)::value * G2_STAGEB;
  };
#endif
  auto dma_step = [&](int st, auto b_) __attribute__((always_inline)) {
    unsigned char* As = stage(b_);
    unsigned char* Bs = As + G2_TILE * 64 * 2;
    const int k0 = kbeg + st * 64;
    // Per-lane offsets are recomputed at every stage (the empty asm hides that
    // they repeat): kept live across the loop for both stages they spill.
    int t = tid;
    if (PROJ_G2_REMAT) __asm__ volatile("" : "+v"(t));
    dma_operand<AK>(A, lda, m0, M, k0, kend, As, t);
    dma_operand<BK>(Bm, ldb, n0, N, k0, kend, Bs, t);
  };

  f32x16 acc[2][4];  // [n block][m block] of C^T
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[nb][mb] = f32x16{};

  // Products of one stage. The fragments of an operand that is not
  // k-contiguous are read with transposing LDS reads, which the compiler
  // cannot tell apart from the copy into the other stage: all of them are
  // read before `start` issues that copy. The plain reads of a k-contiguous
  // operand follow it, one 16-deep sub-step ahead of its products (the
  // scheduling barriers keep the compiler from reading further ahead).
  auto compute = [&](auto b_, auto&& start) __attribute__((always_inline)) {
    const unsigned char* As = stage(b_);
    const unsigned char* Bs = As + G2_TILE * 64 * 2;
    int ln = lane;
    if (PROJ_G2_REMAT) __asm__ volatile("" : "+v"(ln));
    u32x4 af[BK ? 2 : 4][2], bf[AK ? 2 : 4][4];
    auto read = [&](auto kk_, auto tr_) __attribute__((always_inline)) {
      constexpr int kk = decltype(kk_)::value;
      constexpr bool TR = decltype(tr_)::value;
      if constexpr (BK != TR)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) af[BK ? kk & 1 : kk][nb] = frag256<BK>(Bs, wn * 64 + nb * 32, kk, ln);
      if constexpr (AK != TR)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) bf[AK ? kk & 1 : kk][mb] = frag256<AK>(As, wm * 128 + mb * 32, kk, ln);
    };
    static_for<0, 4>([&](auto kk_) __attribute__((always_inline)) { read(kk_, BoolC<true>{}); });
    start();
    read(IntC<0>{}, BoolC<false>{});
    static_for<0, 4>([&](auto kk_) __attribute__((always_inline)) {
      constexpr int kk = decltype(kk_)::value;
      if constexpr (kk + 1 < 4) read(IntC<kk + 1>{}, BoolC<false>{});
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          acc[nb][mb] = E::mfma(af[BK ? kk & 1 : kk][nb], bf[AK ? kk & 1 : kk][mb], acc[nb][mb]);
      if (PROJ_G2_SCHED) __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Stage st in buffer st % 2 (compile-time: the loop takes two stages per
  // iteration); the copy of stage st + 1 runs during the products of stage st.
  // Every stage starts a copy and waits for it on the same path: the last one
  // copies stage nsteps, whose contraction indices all lie at or past kend,
  // so every lane takes the zero offset and no memory is read. (A copy and a
  // wait under separate tests make the compiler assume a copy in flight at
  // the loop head and wait for it before the first LDS read.)
  auto one = [&](int st, auto b_) __attribute__((always_inline)) {
    constexpr int Bf = decltype(b_)::value;
    compute(b_, [&]() __attribute__((always_inline)) { dma_step(st + 1, IntC<Bf ^ 1>{}); });
    wait_vmem();
    __syncthreads();
  };
  dma_step(0, IntC<0>{});
  wait_vmem();
  __syncthreads();
  int st = 0;
  for (; st + 2 <= nsteps; st += 2) {
    one(st, IntC<0>{});
    one(st + 1, IntC<1>{});
  }
  if (st < nsteps) one(st, IntC<0>{});

  // acc[nb][mb][4 j + i] = C[m][n], m = m0 + wm 128 + mb 32 + l32,
  // n = n0 + wn 64 + nb 32 + 8 j + 4 h + i.
  float* slice = S > 1 ? part + (size_t)s * M * N : nullptr;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int m = m0 + wm * 128 + mb * 32 + l32;
    if (m >= M) continue;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 64 + nb * 32 + 8 * j + 4 * h;
        if (n < N) {
          const f32x16& a = acc[nb][mb];
          if (slice) {
            *reinterpret_cast<float4*>(slice + (size_t)m * N + n) =
                make_float4(a[4 * j], a[4 * j + 1], a[4 * j + 2], a[4 * j + 3]);
          } else {
            const u32x2 v = {E::pack(a[4 * j], a[4 * j + 1]), E::pack(a[4 * j + 2], a[4 * j + 3])};
            *reinterpret_cast<u32x2*>(C + (size_t)m * ldc + n) = v;
          }
        }
      }
  }
}

// C[m][n .. n + 3] = sum over s = 0 .. S - 1 (in that order) of the float32
// partial slices, rounded once; one thread per 4 consecutive columns.
template <class E>
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float* __restrict__ part, int S, int M, int N,
                                                            uint16_t* __restrict__ C, int ldc) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const int n4 = N >> 2;
  if (i >= (long)M * n4) return;
  const int m = (int)(i / n4), n = (int)(i - (long)m * n4) * 4;
  const size_t mn = (size_t)M * N, at = (size_t)m * N + n;
  float4 sum = *reinterpret_cast<const float4*>(part + at);
  for (int o = 1; o < S; ++o) {
    const float4 v = *reinterpret_cast<const float4*>(part + o * mn + at);
    sum.x += v.x;
    sum.y += v.y;
    sum.z += v.z;
    sum.w += v.w;
  }
  const u32x2 out = {E::pack(sum.x, sum.y), E::pack(sum.z, sum.w)};
  *reinterpret_cast<u32x2*>(C + (size_t)m * ldc + n) = out;
}

template <class E, bool AK, bool BK, int WM, int WN, int WK>
hipError_t launch_gemm(const uint16_t* A, const uint16_t* Bm, uint16_t* C, int M, int N, int K, int lda, int ldb,
                       int ldc, hipStream_t stream) {
  using S = GemmShape<WM, WN, WK>;
  const int tiles_m = (M + S::BM - 1) / S::BM, tiles_n = (N + S::BN - 1) / S::BN;
  const long total = (long)tiles_m * tiles_n;
  if (total > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_kernel<E, AK, BK, WM, WN, WK>), dim3((unsigned)total), dim3(256), 0, stream, A, Bm, C, M,
                     N, K, lda, ldb, ldc, tiles_n, (int)total);
  return hipGetLastError();
}

// Launch plan of one product. Products with at least 256 rows and columns
// use the 256 x 256 tiles; with a workspace, a product with few such tiles
// splits its contraction until the workgroups about fill the 256 CUs, every
// split keeping at least 8 steps of 64. Smaller products use 128 x 128 tiles
// where there are at least PROJ_MIN_TILES of them, else 64 x 64 tiles with
// the contraction split over the 4 waves.
#ifndef PROJ_MIN_TILES
#define PROJ_MIN_TILES 512
#endif
#ifndef PROJ_BIG
#define PROJ_BIG 1
#endif
#ifndef PROJ_MAX_SPLIT
#define PROJ_MAX_SPLIT 16
#endif
// A product whose 256 x 256 tiles would need a contraction split runs 128 x
// 128 tiles instead, unsplit (no float32 partial slices, no reduction pass),
// when those number at least PROJ_MID_NOSPLIT and the contraction is at most
// PROJ_MID_NOSPLIT_MAXK long. Measured per backward call: B=32, N=196,
// D=768, H=12 (dX: 294 such tiles, K = 2304) 95.4 -> 85.5 us; B=4, N=1024
// 79.1 -> 66.6 us; a long contraction (dW at 32768 tokens, 192 tiles) went
// 456 -> 792 us unsplit, hence the cap.
#ifndef PROJ_MID_NOSPLIT
#define PROJ_MID_NOSPLIT 192
#endif
#ifndef PROJ_MID_NOSPLIT_MAXK
#define PROJ_MID_NOSPLIT_MAXK 4096
#endif

struct GemmPlan {
  bool big;
  int tiles_n, tiles, S, kchunk;
  size_t ws;  // workspace bytes (0 without a split)
};

GemmPlan plan_gemm(int M, int N, int K, bool split_ok) {
  GemmPlan p{};
  p.big = PROJ_BIG && M >= G2_TILE && N >= G2_TILE;
  if (!p.big) return p;
  p.tiles_n = (N + G2_TILE - 1) / G2_TILE;
  const long tiles = (long)((M + G2_TILE - 1) / G2_TILE) * p.tiles_n;
  p.tiles = tiles > INT32_MAX / 16 ? 0 : (int)tiles;  // 0: too many tiles to launch (gemm_auto refuses)
  if (p.tiles == 0) return p;
  p.S = 1;
  if (PROJ_MID_NOSPLIT > 0 && p.tiles < 192 && K <= PROJ_MID_NOSPLIT_MAXK &&
      (long)((M + 127) / 128) * ((N + 127) / 128) >= PROJ_MID_NOSPLIT) {
    p.big = false;  // the 128 x 128 kernel (gemm_auto picks it: at least PROJ_MID_NOSPLIT <= PROJ_MIN_TILES tiles)
    return p;
  }
  if (split_ok && p.tiles < 192) p.S = max(1, min(min(256 / p.tiles, K / 512), PROJ_MAX_SPLIT));
  p.kchunk = ((K + p.S - 1) / p.S + 63) / 64 * 64;
  p.S = (K + p.kchunk - 1) / p.kchunk;
  p.ws = p.S > 1 ? (size_t)p.S * M * N * 4 : 0;
  return p;
}

template <class E, bool AK, bool BK>
hipError_t gemm_auto(const uint16_t* A, const uint16_t* Bm, uint16_t* C, int M, int N, int K, int lda, int ldb,
                     int ldc, void* ws, hipStream_t stream) {
  const GemmPlan p = plan_gemm(M, N, K, ws != nullptr);
  if (p.big && lda <= G2_MAX_LD && ldb <= G2_MAX_LD) {
    if (p.tiles == 0) return hipErrorInvalidValue;
    float* part = p.S > 1 ? static_cast<float*>(ws) : nullptr;
    hipLaunchKernelGGL((gemm256_kernel<E, AK, BK>), dim3((unsigned)(p.tiles * p.S)), dim3(G2_THREADS), 0, stream, A,
                       Bm, C, M, N, K, lda, ldb, ldc, p.tiles_n, p.tiles, p.S, p.kchunk, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.S == 1) return e;
    const long quads = (long)M * (N / 4);
    hipLaunchKernelGGL(reduce_splits_kernel<E>, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, stream, part, p.S,
                       M, N, C, ldc);
    return hipGetLastError();
  }
  const long mid = (long)((M + 127) / 128) * ((N + 127) / 128);
  if (mid >= PROJ_MIN_TILES || (PROJ_MID_NOSPLIT > 0 && mid >= PROJ_MID_NOSPLIT && K <= PROJ_MID_NOSPLIT_MAXK))
    return launch_gemm<E, AK, BK, 2, 2, 1>(A, Bm, C, M, N, K, lda, ldb, ldc, stream);
  return launch_gemm<E, AK, BK, 1, 1, 4>(A, Bm, C, M, N, K, lda, ldb, ldc, stream);
}

template <class E>
hipError_t proj_fwd_e(const uint16_t* x, const uint16_t* w, uint16_t* qkv, long tokens, int D, int HD3,
                      hipStream_t stream) {
  return gemm_auto<E, true, false>(x, w, qkv, (int)tokens, HD3, D, D, HD3, HD3, nullptr, stream);
}

template <class E>
hipError_t proj_bwd_e(const uint16_t* x, const uint16_t* w, const uint16_t* dqkv, uint16_t* dx, uint16_t* dw,
                      long tokens, int D, int HD3, void* ws, hipStream_t stream) {
  hipError_t e = gemm_auto<E, true, true>(dqkv, w, dx, (int)tokens, D, HD3, HD3, HD3, D, ws, stream);
  if (e != hipSuccess) return e;
  return gemm_auto<E, false, false>(x, dqkv, dw, D, HD3, (int)tokens, D, HD3, HD3, ws, stream);
}

}  // namespace

size_t proj_bwd_workspace_bytes(long tokens, int D, int HD3) {
  const size_t a = plan_gemm((int)tokens, D, HD3, true).ws, b = plan_gemm(D, HD3, (int)tokens, true).ws;
  return a > b ? a : b;
}

hipError_t launch_proj_fwd(bool f16, const uint16_t* x, const uint16_t* w, uint16_t* qkv, long tokens, int D, int HD3,
                           hipStream_t stream) {
  return f16 ? proj_fwd_e<F16>(x, w, qkv, tokens, D, HD3, stream) : proj_fwd_e<Bf16>(x, w, qkv, tokens, D, HD3, stream);
}

hipError_t launch_proj_bwd(bool f16, const uint16_t* x, const uint16_t* w, const uint16_t* dqkv, uint16_t* dx,
                           uint16_t* dw, long tokens, int D, int HD3, void* ws, hipStream_t stream) {
  return f16 ? proj_bwd_e<F16>(x, w, dqkv, dx, dw, tokens, D, HD3, ws, stream)
             : proj_bwd_e<Bf16>(x, w, dqkv, dx, dw, tokens, D, HD3, ws, stream);
}

}  // namespace attn
