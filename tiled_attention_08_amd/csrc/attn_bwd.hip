// attn_bwd.hip - recompute-based attention backward for gfx950.
//
// Article "Selbstaufmerksamkeit, CUDA-Kernel und FlashAttention" (German
// edition of the self-attention / Triton / FlashAttention article,
// itimpress.au, 2026-11-15), §3 recompute bullet: the forward keeps only the
// per-row normalisation statistic; the backward rebuilds every probability
// tile on chip from it instead of reading an N x N matrix. The gradient
// formulas are the calculus of the §1 "Attention" formula (the article prints
// none):
//   P = exp(scale Q K^T - lse),  dV = P^T dO,  dP = dO V^T,
//   delta_i = <dO_i, O_i> (= sum_j P_ij dP_ij),  dS = P * (dP - delta),
//   dQ = scale dS K,  dK = scale dS^T Q.
//
// Three launches on one stream, deterministic (no atomics):
//   stage 0  bwd_prep_kernel   workspace <- lse * log2(e) and -delta = -rowsum(dO * O), fp32;
//   stage 1  bwd_dkdv_kernel   one workgroup per (head, 128 keys), looping over
//                              64-query steps: rebuilds S and P, accumulates
//                              dV and dK in registers. A key is a lane column
//                              (S = Q K^T, m = query, n = key), so dV^T = dO^T P
//                              and dK^T = Q^T dS take P and dS straight from
//                              registers; dO^T and Q^T come from transposing
//                              LDS reads of the row-major tiles;
//   stage 2  bwd_dq_kernel     one workgroup per (head, query block), looping
//                              over 32-key steps: rebuilds S^T and P^T with a
//                              query per lane column (lse and delta are then
//                              per-lane scalars) and accumulates dQ^T = K^T dS^T
//                              with dS^T straight from registers.
// The dQ kernel repeats the Q K^T and dO V^T products of the dK/dV kernel: 14
// instead of 10 units of N^2 d work, in exchange for no cross-workgroup
// reduction and no dS round trip through memory.
#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {

namespace {

constexpr int kThreads = 256;
// dK/dV kernel at d_k = 64: 32-query blocks per step and 32-key blocks per
// wave (other head dims: 2 and 1; d_k = 128 has no registers for two key
// blocks, and 32-query tiles of d_k = 32 or 96 would not split evenly over
// the DMA lanes).
#ifndef BWD_FUSE
#define BWD_FUSE 1
#endif
#ifndef BWD_MB64
#define BWD_MB64 2
#endif
#ifndef BWD_KBW64
#define BWD_KBW64 1
#endif
// dQ kernel at d_k <= 64: 32-query blocks per wave (256 or 128 queries per workgroup).
#ifndef BWD_DQ_QB64
#define BWD_DQ_QB64 2
#endif
constexpr int BCQ = 32;                  // dQ kernel: keys per step
// dQ kernel: the dP accumulator starts from -delta (see dq_body). Measured per
// launch: B=8, H=16, N=4096 783 / 778 -> 762 / 761 us, combined launch B=4,
// H=12, N=2048 187 -> 183 us; causal unchanged. dQ rounds differently (the
// sum starts from -delta), within every tolerance of the parity tests.
#ifndef BWD_DQ_DINIT
#define BWD_DQ_DINIT 1
#endif

#ifndef BWD_WAVES_PER_EU
#define BWD_WAVES_PER_EU 2
#endif

// ---------------------------------------------------------------- stage 0: delta
// 8 lanes per row; each lane covers D/8 consecutive elements.
template <class E, int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
                                                       const float* __restrict__ LSE, float* __restrict__ lse2,
                                                       float* __restrict__ ndelta, long rows, int N, int H, Strides so,
                                                       Strides sd) {
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = gid >> 3;
  const int part = (int)(gid & 7);
  constexpr int PER = D / 8;  // elements per lane: 4, 8, 12 or 16, read 4 at a time (8 bytes)
  float s = 0.f;
  if (row < rows) {
    const int bh = (int)(row / N), n = (int)(row - (long)bh * N);
    const uint16_t* o = O + head_off(so, bh, H) + n * so.n + part * PER;
    const uint16_t* g = dO + head_off(sd, bh, H) + n * sd.n + part * PER;
#pragma unroll
    for (int c = 0; c < PER; c += 4) {
      const u32x2 a = *reinterpret_cast<const u32x2*>(o + c);
      const u32x2 b = *reinterpret_cast<const u32x2*>(g + c);
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        s = fmaf(E::lo(a[w]), E::lo(b[w]), s);
        s = fmaf(E::hi(a[w]), E::hi(b[w]), s);
      }
    }
  }
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 4);
  if (row < rows && part == 0) {
    ndelta[row] = -s;
    lse2[row] = LSE[row] * kLog2e;
  }
}

// DMA a row-major [rows x D] block (rows row0.., clamped to N-1) into a
// swizzled LDS tile. Wave `wave` fills `per_lane` runs of 64 consecutive
// 16-byte slots; the lane writing slot (row, s) fetches global chunk
// s ^ swz(row), which yields the layout tile_off() addresses. Rows past N
// re-read row N-1 (finite data); every use of such a row is masked.
// `runs` (total 64-slot runs of the tile) may be below 4 * per_lane: the last
// waves then issue fewer DMAs (callers wait for all of a wave's loads).
template <int D>
__device__ __forceinline__ void dma_rows(Rsrc head_src, int row_stride, int row0, int N, unsigned char* dst, int wave,
                                         int lane, int per_lane, int runs) {
  constexpr int ROWB = D * 2;
  for (int r = 0; r < per_lane; ++r) {
    if (wave * per_lane + r >= runs) break;
    const int slot0 = (wave * per_lane + r) * 64;
    const int p = slot0 + lane;
    const int row = p / (D / 8), chunk = (p - row * (D / 8)) ^ swz<ROWB>(row);
    const int gr = min(row0 + row, N - 1);
    dma16(head_src, (uint32_t)(gr * row_stride + chunk * 8) * 2u, dst + slot0 * 16);
  }
}

// ---------------------------------------------------------------- stage 1: dK, dV
template <int D, int MB>
struct DkdvShape {
  static constexpr int BRQ = 32 * MB;                   // queries per step
  static constexpr int LROWS = BRQ < 64 ? 64 : BRQ;     // lse / -delta entries per buffer (one per DMA lane)
  static constexpr int ROWB = D * 2;
  static constexpr int QTILEB = BRQ * ROWB;             // one Q or dO step tile
  static constexpr int QDMA = BRQ * D / 8 / kThreads;   // 16-byte DMAs per lane per Q or dO tile
  static_assert(QDMA >= 1 && (BRQ * D / 8) % kThreads == 0, "Q / dO tiles split evenly over the lanes");
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_DO = OFF_Q + 2 * QTILEB;
  static constexpr int OFF_L = OFF_DO + 2 * QTILEB;     // lse * log2(e), two buffers
  static constexpr int OFF_DL = OFF_L + 2 * LROWS * 4;  // -delta, two buffers
  static constexpr int LDSB = OFF_DL + 2 * LROWS * 4;
};

// Each wave owns KBW blocks of 32 keys (one key per lane in each), so every
// Q, dO, dO^T and Q^T fragment read from LDS feeds KBW matrix products.
// d_k = 96 and 128, or KBW = 2, need more than 256 registers per lane (the dK
// and dV accumulators alone take 3 to 8 x 16): one wave per SIMD there.
template <class E, int D, int MB, int KBW>
__device__ __forceinline__ void dkdv_body(unsigned char* smem, int work, const uint16_t* __restrict__ Q,
                                          const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                          const uint16_t* __restrict__ dO, const float* __restrict__ lse2,
                                          const float* __restrict__ ndelta, uint16_t* __restrict__ dK,
                                          uint16_t* __restrict__ dV, int N, int n_kblk, int total, float c,
                                          float scale, const int* __restrict__ kv_len, int H, int causal, Strides sq,
                                          Strides sd, Strides sg) {
  using S = DkdvShape<D, MB>;
  constexpr int BRQ = S::BRQ;
  constexpr int BCK = 4 * 32 * KBW;  // keys per workgroup

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int g = lane >> 4, gi = lane & 15;
  const int dsub = g & 1, er = gi >> 2, qq = gi & 3;
  int bh, kblk;  // causal: the first key blocks have the most queries and are handed out first
  work_order(work, total, n_kblk, causal != 0, false, bh, kblk);
  const size_t hq = head_off(sq, bh, H), hd = head_off(sd, bh, H), hg = head_off(sg, bh, H);
  const size_t hrow = (size_t)bh * N;
  const int k0 = kblk * BCK;
  int key[KBW];  // this lane's key in each of its blocks
#pragma unroll
  for (int kb = 0; kb < KBW; ++kb) key[kb] = k0 + (wave * KBW + kb) * 32 + l32;
  // Query i sees key j iff j < kv and (not causal or j <= i); kv = valid keys
  // of this batch entry.
  const int kv = kv_len ? min(max(kv_len[bh / H], 0), N) : N;

  if (k0 >= kv) {  // no query sees any key of this block: zero gradients
#pragma unroll
    for (int kb = 0; kb < KBW; ++kb)
      if (key[kb] < N) {
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int c8 = 0; c8 < D / 8; ++c8) {
          *reinterpret_cast<u32x4*>(dK + hg + key[kb] * sg.n + c8 * 8) = z;
          *reinterpret_cast<u32x4*>(dV + hg + key[kb] * sg.n + c8 * 8) = z;
        }
      }
    return;
  }

  // K and V fragments of this lane's key: B operands of S = Q K^T and dP = dO V^T.
  u32x4 kf[KBW][D / 16], vf[KBW][D / 16];
#pragma unroll
  for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) {
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (key[kb] < N) {
        a = *reinterpret_cast<const u32x4*>(K + hq + key[kb] * sq.n + cc * 16 + h * 8);
        b = *reinterpret_cast<const u32x4*>(V + hq + key[kb] * sq.n + cc * 16 + h * 8);
      }
      kf[kb][cc] = a;
      vf[kb][cc] = b;
    }

  const Rsrc rQ = make_rsrc(Q + hq), rdO = make_rsrc(dO + hd);
  const Rsrc rL = make_rsrc(lse2 + hrow), rDL = make_rsrc(ndelta + hrow);
  auto dma_step = [&](int i, int buf) {
    const int q0 = i * BRQ;
    dma_rows<D>(rQ, sq.n, q0, N, smem + S::OFF_Q + buf * S::QTILEB, wave, lane, S::QDMA, 4 * S::QDMA);
    dma_rows<D>(rdO, sd.n, q0, N, smem + S::OFF_DO + buf * S::QTILEB, wave, lane, S::QDMA, 4 * S::QDMA);
    const uint32_t r = (uint32_t)min(q0 + lane, N - 1) * 4u;
    if (wave == 0) dma4(rL, r, smem + S::OFF_L + buf * S::LROWS * 4);
    if (wave == 1) dma4(rDL, r, smem + S::OFF_DL + buf * S::LROWS * 4);
  };

  f32x16 dvacc[KBW][D / 32], dkacc[KBW][D / 32];
#pragma unroll
  for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      dvacc[kb][db] = f32x16{};
      dkacc[kb][db] = f32x16{};
    }

  // Steps [i_beg, nq) hold a query that sees a key of this block (under the
  // causal mask queries before k0 see none). Steps [u_beg, u_end) need no
  // mask: all their queries exist and see all BCK keys.
  const int nq = (N + BRQ - 1) / BRQ;
  const int i_beg = causal ? k0 / BRQ : 0;
  const int u_beg = causal ? (k0 + BCK - 1 + BRQ - 1) / BRQ : 0;
  const int u_end = k0 + BCK <= kv ? N / BRQ : 0;
  dma_step(i_beg, 0);
  wait_vmem();
  __syncthreads();

  // One 64-query step. MASKED steps give probability 0 to every pair the
  // masks hide (queries or keys past N, keys past kv, keys after the query
  // under the causal mask); other steps carry no masking code.
  // The buffer index is a compile-time constant (BUF == (i - i_beg) % 2) so
  // that every LDS offset in the step folds into an immediate.
  auto step = [&](int i, auto masked, auto bufc) {
    constexpr bool MASKED = decltype(masked)::value;
    constexpr int buf = decltype(bufc)::value;
    const int q0 = i * BRQ;
    if (i + 1 < nq) dma_step(i + 1, buf ^ 1);
    const unsigned char* Qs = smem + S::OFF_Q + buf * S::QTILEB;
    const unsigned char* dOs = smem + S::OFF_DO + buf * S::QTILEB;
    const float* L = reinterpret_cast<const float*>(smem + S::OFF_L + buf * S::LROWS * 4);
    const float* DL = reinterpret_cast<const float*>(smem + S::OFF_DL + buf * S::LROWS * 4);

    // ---- S = Q K^T and dP - delta = dO V^T - delta for BRQ queries x this
    // lane's key. The dP accumulator starts from -delta of its rows (rows
    // 8j + 4h + i, read as four float4 in accumulator order), so no separate
    // subtraction is needed.
    f32x16 sacc[KBW][MB], pacc[KBW][MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      f32x16 dinit;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float4 d4 = *reinterpret_cast<const float4*>(DL + mb * 32 + 8 * jj + 4 * h);
        dinit[4 * jj] = d4.x;
        dinit[4 * jj + 1] = d4.y;
        dinit[4 * jj + 2] = d4.z;
        dinit[4 * jj + 3] = d4.w;
      }
#pragma unroll
      for (int kb = 0; kb < KBW; ++kb) {
        sacc[kb][mb] = f32x16{};
        pacc[kb][mb] = dinit;
      }
#pragma unroll
      for (int cc = 0; cc < D / 16; ++cc) {
        const int off = tile_off<S::ROWB>(mb * 32 + l32, cc * 16 + h * 8);
        const u32x4 aq = lds_read_b128(Qs, off), ado = lds_read_b128(dOs, off);
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) {
          sacc[kb][mb] = E::mfma(aq, kf[kb][cc], sacc[kb][mb]);
          pacc[kb][mb] = E::mfma(ado, vf[kb][cc], pacc[kb][mb]);
        }
      }
    }

    // ---- P = exp2(S * scale * log2 e - lse * log2 e), dS = P * (dP - delta).
    // pp[mb][c2] / dsb[mb][c2]: B operands (bf16 P and dS) for queries mb*32 + 16*c2 + (0..15).
    u32x4 pp[KBW][MB][2], dsb[KBW][MB][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r0 = mb * 32 + 8 * jj + 4 * h;
        const float4 l4 = *reinterpret_cast<const float4*>(L + r0);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb) {
          float p[4], ds[4];
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            p[ii] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][mb][4 * jj + ii], c, -lv[ii]));
            if (MASKED) {
              const int qi = q0 + r0 + ii;
              if (key[kb] >= kv || qi >= N || (causal && key[kb] > qi)) p[ii] = 0.f;
            }
            ds[ii] = p[ii] * pacc[kb][mb][4 * jj + ii];
          }
          const int c2 = jj >> 1, w0 = 2 * (jj & 1);
          pp[kb][mb][c2][w0] = E::pack(p[0], p[1]);
          pp[kb][mb][c2][w0 + 1] = E::pack(p[2], p[3]);
          dsb[kb][mb][c2][w0] = E::pack(ds[0], ds[1]);
          dsb[kb][mb][c2][w0 + 1] = E::pack(ds[2], ds[3]);
        }
      }

    // ---- dV^T += dO^T P and dK^T += Q^T dS (m = dim, n = key, k = query).
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const int row0 = mb * 32 + c2 * 16 + 4 * h + er;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int col = db * 32 + dsub * 16 + 4 * qq;
          const int o0 = tile_off<S::ROWB>(row0, col), o1 = tile_off<S::ROWB>(row0 + 8, col);
          const u32x4 adot = cat(lds_read_tr16_b64(dOs, o0), lds_read_tr16_b64(dOs, o1));
          const u32x4 aqt = cat(lds_read_tr16_b64(Qs, o0), lds_read_tr16_b64(Qs, o1));
#pragma unroll
          for (int kb = 0; kb < KBW; ++kb) {
            dvacc[kb][db] = E::mfma(adot, pp[kb][mb][c2], dvacc[kb][db]);
            dkacc[kb][db] = E::mfma(aqt, dsb[kb][mb][c2], dkacc[kb][db]);
          }
        }
      }

    wait_vmem();
    __syncthreads();  // next step's tiles visible to all waves; this step's buffers free
  };

  // Masked steps before the unmasked range (the causal diagonal), the
  // unmasked range as one single-path loop unrolled by buffer, then the
  // masked steps after it (query tail, or every step when a key of this block
  // is hidden by kv).
  const bool has_u = u_beg < u_end;
  const int m1_end = has_u ? u_beg : nq;
  int i = i_beg;
  for (; i + 1 < m1_end; i += 2) {
    step(i, BoolC<true>{}, IntC<0>{});
    step(i + 1, BoolC<true>{}, IntC<1>{});
  }
  if (i < m1_end) {
    step(i, BoolC<true>{}, IntC<0>{});
    ++i;
  }
  if (has_u) {
    if (i < u_end && ((i - i_beg) & 1)) {
      step(i, BoolC<false>{}, IntC<1>{});
      ++i;
    }
    for (; i + 1 < u_end; i += 2) {
      step(i, BoolC<false>{}, IntC<0>{});
      step(i + 1, BoolC<false>{}, IntC<1>{});
    }
    if (i < u_end) {
      step(i, BoolC<false>{}, IntC<0>{});
      ++i;
    }
    for (; i < nq; ++i) {
      if ((i - i_beg) & 1)
        step(i, BoolC<true>{}, IntC<1>{});
      else
        step(i, BoolC<true>{}, IntC<0>{});
    }
  }

  // ---- epilogue: dV = (dV^T)^T, dK = scale (dK^T)^T, 16-bit RNE. Lane: key, dims db*32 + 8jj + 4h + 0..3.
#pragma unroll
  for (int kb = 0; kb < KBW; ++kb) {
    if (key[kb] >= N) continue;
    uint16_t* dvrow = dV + hg + key[kb] * sg.n;
    uint16_t* dkrow = dK + hg + key[kb] * sg.n;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x16& a = dvacc[kb][db];
        const f32x16& b = dkacc[kb][db];
        const u32x2 wv = {E::pack(a[4 * jj], a[4 * jj + 1]), E::pack(a[4 * jj + 2], a[4 * jj + 3])};
        const u32x2 wk = {E::pack(b[4 * jj] * scale, b[4 * jj + 1] * scale),
                          E::pack(b[4 * jj + 2] * scale, b[4 * jj + 3] * scale)};
        *reinterpret_cast<u32x2*>(dvrow + db * 32 + 8 * jj + 4 * h) = wv;
        *reinterpret_cast<u32x2*>(dkrow + db * 32 + 8 * jj + 4 * h) = wk;
      }
  }
}

template <class E, int D, int MB, int KBW>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(D <= 64 && KBW == 1 ? BWD_WAVES_PER_EU : 1,
                                   D <= 64 && KBW == 1 ? BWD_WAVES_PER_EU : 1)))
void bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                     const uint16_t* __restrict__ dO, const float* __restrict__ lse2, const float* __restrict__ ndelta,
                     uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N, int n_kblk, int total, float c,
                     float scale, const int* __restrict__ kv_len, int H, int causal, Strides sq, Strides sd,
                     Strides sg) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[DkdvShape<D, MB>::LDSB];
  dkdv_body<E, D, MB, KBW>(smem, xcd_remap(blockIdx.x, total), Q, K, V, dO, lse2, ndelta, dK, dV, N, n_kblk, total, c,
                           scale, kv_len, H, causal, sq, sd, sg);
}

// ---------------------------------------------------------------- stage 1, software-pipelined (d_k = 64)
// The dK/dV kernel above runs each 64-query step as three dependent phases
// (S and dP products, then the exponentials, then the dV and dK products), so
// a wave's matrix products and its vector ALU work never overlap; the other
// wave on the SIMD is left to fill the gaps, which it does poorly (a wave
// issuing exponentials slows a neighbour's matrix products far more than the
// same exponentials interleaved in the product stream of one wave). This
// variant is for the unmasked case with N a multiple of 64 and d_k = 64 (the
// long-sequence shapes). It splits a step into two 32-query units
// and runs one slot per unit: the slot of unit t issues the dV and dK products
// of unit t - 1 and the S and dP products of unit t + 1 while computing P and
// dS of unit t from the S and dP accumulators of the previous slot. Each of
// the 16 chunks of a slot holds one matrix product, one exponential and its
// fma, multiply and half a pack. Same arithmetic in the same order as the
// kernel above: bit-identical results. Measured at B=8, H=16, N=4096: 997.6
// -> 987.3 us with a ring of 3 step tiles (4: 989.3 us; operands read 1, 2
// or 3 products ahead: 1044.5, 987.3, 987.6 us); matrix-core busy time stays
// near 60 % of the cycles. The products' power draw with random operands,
// not the instruction schedule, sets the pace.
#ifndef BWD_SP
#define BWD_SP 1
#endif
#ifndef BWD_SP_RING
#define BWD_SP_RING 3
#endif
// Waves per workgroup (32 keys each), all sharing each Q / dO step tile. 8
// waves (one workgroup per CU, half the tile copies per key) measured no
// faster: B=8, H=16, N=4096 973 -> 983-990 us, B=4, H=12, N=2048 103 -> 119 us.
#ifndef BWD_SP_WAVES
#define BWD_SP_WAVES 4
#endif
#ifndef BWD_SP_AHEAD
#define BWD_SP_AHEAD 2
#endif
// Causal rows on the pipelined dK/dV kernel (d_k = 64, N a multiple of 128;
// bit-identical to the single-phase kernel): B=8, H=16, N=4096 537-547 ->
// 513-522 us, B=4, H=12, N=2048 67-74 -> 62 us, B=2, H=16, N=8192 509-511 ->
// 500-501 us.
#ifndef BWD_SP_CAUSAL
#define BWD_SP_CAUSAL 1
#endif
// BWD_SP_PIN keeps each chunk's exponentials in the chunk (see the slot
// body). Measured, bit-identical outputs: B=8, H=16, N=4096 977 -> 957-962
// us, B=2, H=16, N=8192 969 -> 951 us.
#ifndef BWD_SP_PIN
#define BWD_SP_PIN 1
#endif
// Chunks of a slot that read the next unit's -delta and lse.
#ifndef BWD_SP_DLREAD
#define BWD_SP_DLREAD 4
#endif
#ifndef BWD_SP_LREAD
#define BWD_SP_LREAD 12
#endif

template <int WAVES>
struct DkdvSpShape {
  static constexpr int D = 64, BRQ = 64, ROWB = 2 * D, THREADS = 64 * WAVES;
  static constexpr int BCK = 32 * WAVES;               // keys per workgroup (32 per wave)
  static constexpr int QTILEB = BRQ * ROWB;            // one Q or dO step tile (8 KB)
  static constexpr int QDMA = BRQ * D / 8 / THREADS;   // 16-byte DMAs per lane per tile (2 with 4 waves, 1 with 8)
  static_assert(QDMA >= 1 && (BRQ * D / 8) % THREADS == 0, "step tiles split evenly over the lanes");
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_DO = QTILEB;
  static constexpr int OFF_L = 2 * QTILEB;             // lse * log2(e) of the step's 64 queries
  static constexpr int OFF_DL = OFF_L + BRQ * 4;       // -delta
  static constexpr int SLOTB = OFF_DL + BRQ * 4;       // one ring slot
};

// The ring slots of the pipelined dK/dV body: one LDS array each, declared by
// the kernel, so that the compiler sees that the copy into one slot cannot
// alias the reads of another.
struct SpRing {
  unsigned char* s[4];
};

// RAG: 0 when N is a multiple of the 64-query step; otherwise rows past N
// are read as row N - 1 and get probability 0 in the last step, whose second
// 32-query unit holds rows (RAG 1: N % 64 above 32) or none (RAG 2: that unit,
// whose P and dS would all be 0, is not computed). Measured for RAG 2
// (identical results): B=32, H=12, N=196 combined launch 35.1-38.0 -> 33.6-35.8
// us, B=16, H=12, N=197 19.7-20.8 -> 18.7-19.9 us.
inline int dkdv_rag_of(int N) { return N % 64 == 0 ? 0 : (N % 64 <= 32 ? 2 : 1); }

// CAUSAL (N a multiple of 128): the body starts at the first step whose
// queries see a key of the block, and masks its first two steps (the
// diagonal: P and dS are 0 for a key after the query), as dkdv_body does;
// blocks are handed out heaviest first.
template <class E, int NS, int WAVES, int RAG, bool CAUSAL>
__device__ __forceinline__ void dkdv_sp_body(const SpRing& ring, int work, const uint16_t* __restrict__ Q,
                                             const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                             const uint16_t* __restrict__ dO, const float* __restrict__ lse2,
                                             const float* __restrict__ ndelta, uint16_t* __restrict__ dK,
                                             uint16_t* __restrict__ dV, int N, int n_kblk, int total, float c,
                                             float scale, int H, Strides sq, Strides sd, Strides sg) {
  using S = DkdvSpShape<WAVES>;
  constexpr int D = S::D;
  static_assert(NS == 3 || NS == 4, "ring of 3 or 4 step tiles");
  auto slot_base = [&](auto r_) __attribute__((always_inline)) -> unsigned char* {
    constexpr int R = decltype(r_)::value % NS;
    return ring.s[R];
  };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int g = lane >> 4, gi = lane & 15;
  const int dsub = g & 1, er = gi >> 2, qq = gi & 3;
  int bh, kblk;
  work_order(work, total, n_kblk, CAUSAL, false, bh, kblk);
  const size_t hq = head_off(sq, bh, H), hd = head_off(sd, bh, H), hg = head_off(sg, bh, H);
  const size_t hrow = (size_t)bh * N;
  const int key = kblk * S::BCK + wave * 32 + l32;  // this lane's key (keys past N compute unused gradients)
  // Steps i of the body are query steps s0 + i (s0 = 0 without the mask).
  const int s0 = CAUSAL ? kblk * S::BCK / S::BRQ : 0;

  u32x4 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (key < N) {
      a = *reinterpret_cast<const u32x4*>(K + hq + key * sq.n + cc * 16 + h * 8);
      b = *reinterpret_cast<const u32x4*>(V + hq + key * sq.n + cc * 16 + h * 8);
    }
    kf[cc] = a;
    vf[cc] = b;
  }

  const Rsrc rQ = make_rsrc(Q + hq), rdO = make_rsrc(dO + hd);
  const Rsrc rL = make_rsrc(lse2 + hrow), rDL = make_rsrc(ndelta + hrow);
  // DMA counts per tile: 2 * QDMA for every wave, one more for waves 0 and 1.
  constexpr int PER = 2 * S::QDMA;
  // Ragged: rows past N repeat row N - 1 (finite data, whose probabilities
  // the last step sets to 0).
  auto dma_tile = [&](int i, auto r_) __attribute__((always_inline)) {
    unsigned char* base = slot_base(r_);
    const int q0 = (s0 + i) * S::BRQ;
#pragma unroll
    for (int r = 0; r < S::QDMA; ++r) {
      const int slot0 = (wave * S::QDMA + r) * 64;
      const int p = slot0 + lane;
      const int row = p / (D / 8), chunk = (p - row * (D / 8)) ^ swz<S::ROWB>(row);
      const int qr = RAG ? min(q0 + row, N - 1) : q0 + row;
      dma16(rQ, (uint32_t)(qr * sq.n + chunk * 8) * 2u, base + S::OFF_Q + slot0 * 16);
      dma16(rdO, (uint32_t)(qr * sd.n + chunk * 8) * 2u, base + S::OFF_DO + slot0 * 16);
    }
    const uint32_t lr = (uint32_t)(RAG ? min(q0 + lane, N - 1) : q0 + lane) * 4u;
    if (wave == 0) dma4(rL, lr, base + S::OFF_L);
    if (wave == 1) dma4(rDL, lr, base + S::OFF_DL);
  };

  // Per-lane LDS offsets (query block 0, 16-query half 0; the other blocks
  // and halves add whole rows, which leave the swizzle unchanged).
  int koff[D / 16], toff[2][2];
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) koff[cc] = tile_off<S::ROWB>(l32, cc * 16 + h * 8);
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) toff[db][hi] = tile_off<S::ROWB>(4 * h + er + 8 * hi, db * 32 + dsub * 16 + 4 * qq);

  // Product m of a slot: m < 8 the dV / dK products of the previous unit
  // (kind m & 1: dV^T += dO^T P or dK^T += Q^T dS; 32-dim block (m >> 1) & 1;
  // 16-query half m >> 2), m >= 8 the S / dP products of the next unit
  // (b = m - 8: kind b & 1: S = Q K^T or dP = dO V^T; 16-dim chunk b >> 1).
  // Operand of product m: transposed dO or Q fragment, or a Q or dO fragment.
  auto operand = [&](int m, auto ra_, auto mba_, auto rb_, auto mbb_) __attribute__((always_inline)) -> u32x4 {
    if (m < 8) {
      const unsigned char* T = slot_base(ra_) + ((m & 1) ? S::OFF_Q : S::OFF_DO);
      const int rows = (decltype(mba_)::value * 32 + (m >> 2) * 16) * S::ROWB, db = (m >> 1) & 1;
      return cat(lds_read_tr16_b64(T, rows + toff[db][0]), lds_read_tr16_b64(T, rows + toff[db][1]));
    }
    const int b = m - 8;
    const unsigned char* T = slot_base(rb_) + ((b & 1) ? S::OFF_DO : S::OFF_Q);
    return lds_read_b128(T, decltype(mbb_)::value * 32 * S::ROWB + koff[b >> 1]);
  };

  f32x16 dvacc[2], dkacc[2];
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    dvacc[db] = f32x16{};
    dkacc[db] = f32x16{};
  }

  // One slot. A (HA): dV / dK products of the unit in query block MBA of the
  // tile in ring slot RA, from its bf16 P and dS in ya / yd. B (HB): S and
  // dP - delta of the unit in query block MBB of the tile in slot RB into sn
  // / pn, and that unit's lse into ln. V (HV): P and dS of the current unit
  // from sv / pv and lse lv into xp / xd (pair i of entries 2i, 2i + 1 goes
  // to word i & 3 of operand i >> 2).
  auto slot = [&](auto hasA, auto ra_, auto mba_, const u32x4 (&ya)[2], const u32x4 (&yd)[2], auto hasB, auto rb_,
                  auto mbb_, f32x16& sn, f32x16& pn, float (&ln)[16], auto hasV, const f32x16& sv, const f32x16& pv,
                  const float (&lv)[16], u32x4 (&xp)[2], u32x4 (&xd)[2], auto maskV, int qv0)
                  __attribute__((always_inline)) {
    // maskV: the current unit (first query qv0) has rows past N, whose P and dS are 0.
    constexpr bool HA = decltype(hasA)::value, HB = decltype(hasB)::value, HV = decltype(hasV)::value;
    constexpr bool MV = decltype(maskV)::value;
    constexpr int MBB = decltype(mbb_)::value;
    constexpr int AH = BWD_SP_AHEAD, NO = AH + 1;
    constexpr int M0 = HA ? 0 : 8, M1 = HB ? 16 : 8;  // products [M0, M1)
    u32x4 ops[NO];
    static_for<0, AH>([&](auto a_) __attribute__((always_inline)) {
      constexpr int m = M0 + decltype(a_)::value;
      if constexpr (m < M1) ops[m % NO] = operand(m, ra_, mba_, rb_, mbb_);
    });
    float pe = 0.f, de = 0.f;  // P and dS of the even entry of the pair
    static_for<0, 16>([&](auto k_) __attribute__((always_inline)) {
      constexpr int KK = decltype(k_)::value;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (HB && KK == BWD_SP_DLREAD) {
        // -delta of the next unit's rows (8j + 4h + i) starts its dP accumulator.
        const float* DL = reinterpret_cast<const float*>(slot_base(rb_) + S::OFF_DL) + MBB * 32 + 4 * h;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float4 d4 = *reinterpret_cast<const float4*>(DL + 8 * jj);
          pn[4 * jj] = d4.x;
          pn[4 * jj + 1] = d4.y;
          pn[4 * jj + 2] = d4.z;
          pn[4 * jj + 3] = d4.w;
        }
      }
      if constexpr (HB && KK == BWD_SP_LREAD) {
        const float* L = reinterpret_cast<const float*>(slot_base(rb_) + S::OFF_L) + MBB * 32 + 4 * h;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float4 l4 = *reinterpret_cast<const float4*>(L + 8 * jj);
          ln[4 * jj] = l4.x;
          ln[4 * jj + 1] = l4.y;
          ln[4 * jj + 2] = l4.z;
          ln[4 * jj + 3] = l4.w;
        }
      }
      if constexpr (KK >= M0 && KK < M1) {
        if constexpr (KK < 8) {
          constexpr int db = (KK >> 1) & 1, c2 = KK >> 2;
          if constexpr (KK & 1)
            dkacc[db] = E::mfma(ops[KK % NO], yd[c2], dkacc[db]);
          else
            dvacc[db] = E::mfma(ops[KK % NO], ya[c2], dvacc[db]);
        } else {
          constexpr int b = KK - 8, cc = b >> 1;
          if constexpr (b == 0) sn = f32x16{};
          if constexpr (b & 1)
            pn = E::mfma(ops[KK % NO], vf[cc], pn);
          else
            sn = E::mfma(ops[KK % NO], kf[cc], sn);
        }
      }
      if constexpr (KK >= M0 && KK + AH < M1) ops[(KK + AH) % NO] = operand(KK + AH, ra_, mba_, rb_, mbb_);
      if constexpr (HV) {
        float p = __builtin_amdgcn_exp2f(fmaf(sv[KK], c, -lv[KK]));
        if constexpr (MV) {
          const int qr = qv0 + 8 * (KK >> 2) + 4 * h + (KK & 3);
          if ((RAG != 0 && qr >= N) || (CAUSAL && qr < key)) p = 0.f;
        }
        const float ds = p * pv[KK];
        if constexpr (KK & 1) {
          constexpr int i = KK >> 1;
          xp[i >> 2][i & 3] = E::pack(pe, p);
          xd[i >> 2][i & 3] = E::pack(de, ds);
#if BWD_SP_PIN
          // Empty uses keep this pair's exponentials in this chunk: P and dS
          // are first read by the next slot, and the compiler otherwise moves
          // a whole slot's vector work away from its products.
          __asm__ volatile("" : : "v"(xp[i >> 2][i & 3]), "v"(xd[i >> 2][i & 3]));
#endif
        } else {
          pe = p;
          de = ds;
        }
      }
    });
    __builtin_amdgcn_sched_barrier(0);
  };

  // Steps (the launcher checks that there are at least NS, or under the
  // causal mask at least 2: N is then a multiple of 128).
  const int nq = (N + S::BRQ - 1) / S::BRQ - s0;
  // Before the slot of unit (i, 1): tile i + 1 landed and visible to every
  // wave, every wave done with tile i - 1, whose ring slot takes tile
  // i - 1 + NS.
  auto boundary = [&](int i, auto r_) __attribute__((always_inline)) {
    constexpr int R = decltype(r_)::value;
    if (i + 1 >= nq) return;
    if constexpr (NS == 4) {
      if (i + 2 < nq)
        wait_vmem_below<PER>();
      else
        wait_vmem_below<0>();
    } else {
      wait_vmem_below<0>();
    }
    __syncthreads();
    if (i - 1 + NS < nq) dma_tile(i - 1 + NS, IntC<(R + NS - 1) % NS>{});
  };

  f32x16 s_0, g_0, s_1, g_1;          // S and dP - delta of the current units of query blocks 0 and 1
  float l_0[16], l_1[16];             // their lse * log2(e)
  u32x4 wp_0[2], wd_0[2], wp_1[2], wd_1[2];  // bf16 P and dS of query blocks 0 and 1
  // Step i in ring slot R: the slots of units (i, 0) and (i, 1). MASK: the
  // step holds rows past N (the last step of a ragged sequence).
  auto step = [&](int i, auto r_, auto first_, auto last_, auto mask_) __attribute__((always_inline)) {
    constexpr int R = decltype(r_)::value;
    constexpr bool FIRST = decltype(first_)::value, LAST = decltype(last_)::value;
    // unit (i, 0): dV / dK of (i - 1, 1), S / dP of (i, 1), P / dS of (i, 0)
    slot(BoolC<!FIRST>{}, IntC<(R + NS - 1) % NS>{}, IntC<1>{}, wp_1, wd_1, BoolC<true>{}, r_, IntC<1>{}, s_1, g_1, l_1,
         BoolC<true>{}, s_0, g_0, l_0, wp_0, wd_0, mask_, (s0 + i) * S::BRQ);
    boundary(i, r_);
    // unit (i, 1): dV / dK of (i, 0), S / dP of (i + 1, 0), P / dS of (i, 1)
    slot(BoolC<true>{}, r_, IntC<0>{}, wp_0, wd_0, BoolC<!LAST>{}, IntC<(R + 1) % NS>{}, IntC<0>{}, s_0, g_0, l_0,
         BoolC<true>{}, s_1, g_1, l_1, wp_1, wd_1, mask_, (s0 + i) * S::BRQ + 32);
  };

  // Prologue: tiles 0 .. NS - 2 in flight, tile 0 resident, S / dP of unit (0, 0).
  static_for<0, NS - 1>([&](auto r_) __attribute__((always_inline)) { dma_tile(decltype(r_)::value, r_); });
  wait_vmem_below<0>();
  __syncthreads();
  slot(BoolC<false>{}, IntC<0>{}, IntC<0>{}, wp_1, wd_1, BoolC<true>{}, IntC<0>{}, IntC<0>{}, s_0, g_0, l_0,
       BoolC<false>{}, s_1, g_1, l_1, wp_0, wd_0, BoolC<false>{}, 0);
  // Steps 0 .. nq - 2, NS per iteration (compile-time ring slots), then the
  // rest and the last step, and the dV / dK of the last unit.
  // Under the causal mask steps 0 and 1 are the diagonal (masked); step 1
  // is the last step when there are two.
  step(0, IntC<0>{}, BoolC<true>{}, BoolC<false>{}, BoolC<CAUSAL>{});
  constexpr int I0 = CAUSAL ? 2 : 1;  // first step of the loop below
  if constexpr (CAUSAL) {
    if (nq > 2) step(1, IntC<1>{}, BoolC<false>{}, BoolC<false>{}, BoolC<true>{});
  }
  int i = I0;
  for (; i + NS <= nq - 1; i += NS) {
    static_for<0, NS>([&](auto u_) __attribute__((always_inline)) {
      step(i + decltype(u_)::value, IntC<(I0 + decltype(u_)::value) % NS>{}, BoolC<false>{}, BoolC<false>{},
           BoolC<false>{});
    });
  }
  static_for<0, NS - 1>([&](auto u_) __attribute__((always_inline)) {
    constexpr int U = decltype(u_)::value;
    if (i + U < nq - 1) step(i + U, IntC<(I0 + U) % NS>{}, BoolC<false>{}, BoolC<false>{}, BoolC<false>{});
  });
  // The last step, nq - 1, in ring slot (nq - 1) % NS, with the row mask when
  // ragged (a template parameter: a second, runtime-selected copy of the step
  // pushes the kernel over 256 registers). With RAG 2 its second unit has no
  // rows: the step is the slot of its first unit without the next unit's
  // products, then the dV / dK products of that first unit.
  static_for<0, NS>([&](auto r_) __attribute__((always_inline)) {
    constexpr int R = decltype(r_)::value;
    if ((nq - 1) % NS == R) {
      if constexpr (RAG == 2) {
        slot(BoolC<true>{}, IntC<(R + NS - 1) % NS>{}, IntC<1>{}, wp_1, wd_1, BoolC<false>{}, r_, IntC<1>{}, s_1, g_1,
             l_1, BoolC<true>{}, s_0, g_0, l_0, wp_0, wd_0, BoolC<true>{}, (s0 + nq - 1) * S::BRQ);
        slot(BoolC<true>{}, r_, IntC<0>{}, wp_0, wd_0, BoolC<false>{}, r_, IntC<0>{}, s_0, g_0, l_0, BoolC<false>{},
             s_1, g_1, l_1, wp_1, wd_1, BoolC<false>{}, 0);
      } else {
        step(nq - 1, r_, BoolC<false>{}, BoolC<true>{}, BoolC<(RAG != 0 || CAUSAL)>{});
        slot(BoolC<true>{}, r_, IntC<1>{}, wp_1, wd_1, BoolC<false>{}, r_, IntC<0>{}, s_0, g_0, l_0, BoolC<false>{}, s_1,
             g_1, l_1, wp_0, wd_0, BoolC<false>{}, 0);
      }
    }
  });

  // Epilogue: dV = (dV^T)^T, dK = scale (dK^T)^T, 16-bit RNE. Lane: key, dims db*32 + 8jj + 4h + 0..3.
  if (key < N) {
    uint16_t* dvrow = dV + hg + key * sg.n;
    uint16_t* dkrow = dK + hg + key * sg.n;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x16& a = dvacc[db];
        const f32x16& b = dkacc[db];
        const u32x2 wv = {E::pack(a[4 * jj], a[4 * jj + 1]), E::pack(a[4 * jj + 2], a[4 * jj + 3])};
        const u32x2 wk = {E::pack(b[4 * jj] * scale, b[4 * jj + 1] * scale),
                          E::pack(b[4 * jj + 2] * scale, b[4 * jj + 3] * scale)};
        *reinterpret_cast<u32x2*>(dvrow + db * 32 + 8 * jj + 4 * h) = wv;
        *reinterpret_cast<u32x2*>(dkrow + db * 32 + 8 * jj + 4 * h) = wk;
      }
  }
}

template <class E, int NS, int WAVES, int RAG, bool CAUSAL>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_sp_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                        const uint16_t* __restrict__ dO, const float* __restrict__ lse2,
                        const float* __restrict__ ndelta, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N,
                        int n_kblk, int total, float c, float scale, int H, Strides sq, Strides sd, Strides sg) {
  using S = DkdvSpShape<WAVES>;
  __shared__ __attribute__((aligned(16))) unsigned char ring0[S::SLOTB];
  __shared__ __attribute__((aligned(16))) unsigned char ring1[S::SLOTB];
  __shared__ __attribute__((aligned(16))) unsigned char ring2[S::SLOTB];
  __shared__ __attribute__((aligned(16))) unsigned char ring3[NS == 4 ? S::SLOTB : 16];
  dkdv_sp_body<E, NS, WAVES, RAG, CAUSAL>(SpRing{{ring0, ring1, ring2, ring3}}, xcd_remap(blockIdx.x, total), Q, K,
                                          V, dO, lse2, ndelta, dK, dV, N, n_kblk, total, c, scale, H, sq, sd, sg);
}

// ---------------------------------------------------------------- stage 2: dQ
template <int D, int QB>
struct DqShape {
  static constexpr int BR = 4 * 32 * QB;                // queries per workgroup
  static constexpr int ROWB = D * 2;
  static constexpr int TILEB = BCQ * ROWB;              // one K or V step tile
  static constexpr int KRUNS = BCQ * D / 8 / 64;        // 64-slot DMA runs per K or V tile (2 to 8)
  static constexpr int KDMA = (KRUNS + 3) / 4;          // runs per wave (the last waves may do fewer)
  static constexpr int BUFB = 2 * TILEB;                // one buffer: K and V of a step
};

// buf0, buf1: the two step buffers (K tile, then V tile), separate LDS arrays
// so that the compiler can tell the DMA into one from the transposing reads
// of the other (otherwise those reads wait for the step in flight).
template <class E, int D, int QB>
__device__ __forceinline__ void dq_body(unsigned char* buf0, unsigned char* buf1, int work, const uint16_t* __restrict__ Q,
                                        const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                        const uint16_t* __restrict__ dO, const float* __restrict__ lse2_in,
                                        const float* __restrict__ ndelta, uint16_t* __restrict__ dQ, int N,
                                        int n_qblk, int total, float c, float scale, const int* __restrict__ kv_len,
                                        int H, int causal, Strides sq, Strides sd, Strides sg) {
  using S = DqShape<D, QB>;
  static_assert((BCQ * D / 8) % 64 == 0, "K/V step tiles are whole 64-slot runs");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int g = lane >> 4, gi = lane & 15;
  const int dsub = g & 1, er = gi >> 2, qq = gi & 3;
  int bh, qblk;  // causal: the last row blocks have the most keys and are handed out first
  work_order(work, total, n_qblk, causal != 0, true, bh, qblk);
  const size_t hq = head_off(sq, bh, H), hd = head_off(sd, bh, H);
  const size_t hrow = (size_t)bh * N;
  const int qw0 = qblk * S::BR + wave * 32 * QB;

  // Visible keys of query q: j < klim(q) = min(kv, q + 1) (causal) or kv.
  const int kv = kv_len ? min(max(kv_len[bh / H], 0), N) : N;
  auto klim = [&](int q) { return causal ? min(kv, q + 1) : kv; };
  int klq[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) klq[qb] = klim(qw0 + qb * 32 + l32);
  // Key steps this workgroup reads, steps all its queries see in full, and
  // the steps this wave has any visible key in.
  const int ntiles = (klim(qblk * S::BR + S::BR - 1) + BCQ - 1) / BCQ;
  const int nfull = klim(qblk * S::BR) / BCQ;
  const int nvis_w = (klim(qw0 + 32 * QB - 1) + BCQ - 1) / BCQ;

  // Per query (lane column l32 of block qb): Q and dO fragments (B operands of
  // S^T = K Q^T and dP^T = V dO^T), lse in log2 units and -delta.
  u32x4 qf[QB][D / 16], df[QB][D / 16];
  float lse2[QB], dl[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int q = qw0 + qb * 32 + l32;
    const bool ok = q < N;
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) {
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (ok) {
        a = *reinterpret_cast<const u32x4*>(Q + hq + q * sq.n + cc * 16 + h * 8);
        b = *reinterpret_cast<const u32x4*>(dO + hd + q * sd.n + cc * 16 + h * 8);
      }
      qf[qb][cc] = a;
      df[qb][cc] = b;
    }
    lse2[qb] = ok ? lse2_in[hrow + q] : 0.f;
    dl[qb] = ok ? ndelta[hrow + q] : 0.f;
  }

  f32x16 dqacc[QB][D / 32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) dqacc[qb][db] = f32x16{};

  const Rsrc rK = make_rsrc(K + hq), rV = make_rsrc(V + hq);
  auto dma_step = [&](int j, auto buf_c) {
    unsigned char* dst = decltype(buf_c)::value ? buf1 : buf0;
    dma_rows<D>(rK, sq.n, j * BCQ, N, dst, wave, lane, S::KDMA, S::KRUNS);
    dma_rows<D>(rV, sq.n, j * BCQ, N, dst + S::TILEB, wave, lane, S::KDMA, S::KRUNS);
  };

  if (ntiles > 0) {
    dma_step(0, IntC<0>{});
    wait_vmem();
  }
  __syncthreads();

  // Per-lane byte offsets of the operand reads within a step tile: K and V
  // rows l32 (chunk 2cc + h), and the transposing K reads of rows 4h + er
  // (+ 8). The swizzle depends only on a row's low 4 bits, so the 16-row
  // halves and the buffer are immediate offsets of the reads.
  int koff[D / 16], toff[2][D / 32];
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) koff[cc] = tile_off<S::ROWB>(l32, cc * 16 + h * 8);
#pragma unroll
  for (int hi = 0; hi < 2; ++hi)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) toff[hi][db] = tile_off<S::ROWB>(4 * h + er + 8 * hi, db * 32 + dsub * 16 + 4 * qq);

  // One 32-key step. MASKED steps give probability 0 to each lane's keys at
  // or beyond klim(query) (keys past N or kv, keys after the query under the
  // causal mask). COMPUTE false: this wave sees no key of the step and only
  // takes part in the DMA. BUF (= j & 1) is a compile-time constant.
  auto step = [&](int j, auto masked, bool compute, auto bufc) {
    constexpr bool MASKED = decltype(masked)::value;
    constexpr int buf = decltype(bufc)::value;
    if (j + 1 < ntiles) dma_step(j + 1, IntC<buf ^ 1>{});
    if (!compute) return;
    const unsigned char* Ks = buf ? buf1 : buf0;
    const unsigned char* Vs = Ks + S::TILEB;

    // ---- S^T = K Q^T and dP^T - delta = V dO^T - delta: 32 keys x (32*QB)
    // queries. With BWD_DQ_DINIT the dP accumulator starts from -delta of its
    // query (every entry of a lane column), as the dK/dV kernel's does, which
    // saves an add per entry.
    f32x16 sacc[QB], pacc[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      sacc[qb] = f32x16{};
#pragma unroll
      for (int e = 0; e < 16; ++e) pacc[qb][e] = BWD_DQ_DINIT ? dl[qb] : 0.f;
    }
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) {
      const u32x4 ak = lds_read_b128(Ks, koff[cc]);
      const u32x4 av = lds_read_b128(Vs, koff[cc]);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        sacc[qb] = E::mfma(ak, qf[qb][cc], sacc[qb]);
        pacc[qb] = E::mfma(av, df[qb][cc], pacc[qb]);
      }
    }

    // ---- dS^T = P^T * (dP^T - delta), P^T = exp2(S^T c - lse2); packed as the
    // B operand of dQ^T = K^T dS^T for keys 16*c2 + (0..15).
    u32x4 dsb[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[qb][e], c, -lse2[qb]));
        float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[qb][e + 1], c, -lse2[qb]));
        if (MASKED) {
          const int key = j * BCQ + 8 * (e >> 2) + 4 * h + (e & 3);
          if (key >= klq[qb]) p0 = 0.f;
          if (key + 1 >= klq[qb]) p1 = 0.f;
        }
        const float g0 = BWD_DQ_DINIT ? pacc[qb][e] : pacc[qb][e] + dl[qb];
        const float g1 = BWD_DQ_DINIT ? pacc[qb][e + 1] : pacc[qb][e + 1] + dl[qb];
        dsb[qb][e >> 3][(e >> 1) & 3] = E::pack(p0 * g0, p1 * g1);
      }

    // ---- dQ^T += K^T dS^T (m = dim, n = query, k = key); K^T by transposing reads.
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const u32x4 a = cat(lds_read_tr16_b64(Ks, c2 * 16 * S::ROWB + toff[0][db]),
                            lds_read_tr16_b64(Ks, c2 * 16 * S::ROWB + toff[1][db]));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) dqacc[qb][db] = E::mfma(a, dsb[qb][c2], dqacc[qb][db]);
      }
    }
  };

  // Steps all queries see in full, two per iteration (buffers 0 and 1), then the rest.
  int j = 0;
  for (; j + 1 < nfull; j += 2) {
    step(j, BoolC<false>{}, true, IntC<0>{});
    wait_vmem();
    __syncthreads();
    step(j + 1, BoolC<false>{}, true, IntC<1>{});
    wait_vmem();
    __syncthreads();
  }
  if (j < nfull) {  // j even
    step(j, BoolC<false>{}, true, IntC<0>{});
    wait_vmem();
    __syncthreads();
    ++j;
  }
  for (; j < ntiles; ++j) {
    if (j & 1)
      step(j, BoolC<true>{}, j < nvis_w, IntC<1>{});
    else
      step(j, BoolC<true>{}, j < nvis_w, IntC<0>{});
    if (j + 1 < ntiles) {
      wait_vmem();
      __syncthreads();
    }
  }

  // ---- epilogue: dQ = scale (dQ^T)^T, bf16 RNE. Lane: query, dims db*32 + 8jj + 4h + 0..3.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int q = qw0 + qb * 32 + l32;
    if (q < N) {
      uint16_t* row = dQ + head_off(sg, bh, H) + q * sg.n;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x16& a = dqacc[qb][db];
          const u32x2 w = {E::pack(a[4 * jj] * scale, a[4 * jj + 1] * scale),
                           E::pack(a[4 * jj + 2] * scale, a[4 * jj + 3] * scale)};
          *reinterpret_cast<u32x2*>(row + db * 32 + 8 * jj + 4 * h) = w;
        }
    }
  }
}

// One 32-query block per wave at d_k = 64 (156 registers) runs three waves
// per SIMD; used for causal rows (BWD_DQ_CAUSAL_QB1).
constexpr int dq_waves_per_eu(int D, int QB) { return D == 64 && QB == 1 ? 3 : BWD_WAVES_PER_EU; }

template <class E, int D, int QB>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(dq_waves_per_eu(D, QB), dq_waves_per_eu(D, QB))))
void bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                   const uint16_t* __restrict__ dO, const float* __restrict__ lse2_in, const float* __restrict__ ndelta,
                   uint16_t* __restrict__ dQ, int N, int n_qblk, int total, float c, float scale,
                   const int* __restrict__ kv_len, int H, int causal, Strides sq, Strides sd, Strides sg) {
  __shared__ __attribute__((aligned(16))) unsigned char buf0[DqShape<D, QB>::BUFB];
  __shared__ __attribute__((aligned(16))) unsigned char buf1[DqShape<D, QB>::BUFB];
  dq_body<E, D, QB>(buf0, buf1, xcd_remap(blockIdx.x, total), Q, K, V, dO, lse2_in, ndelta, dQ, N, n_qblk, total, c, scale,
                    kv_len, H, causal, sq, sd, sg);
}

// ---------------------------------------------------------------- stage 2, software-pipelined (d_k = 64)
// The dQ kernel above runs each 32-key step as three dependent phases (S^T
// and dP^T products, then the exponentials, then the dQ^T products), so a
// wave's products and its vector work overlap only with the other wave of
// its SIMD. This variant (unmasked rows, N a multiple of 64, d_k = 64) gives
// each wave one 32-query block and runs one slot per 32-key unit: the slot of
// unit u issues the dQ^T products of unit u - 1 and the S^T and dP^T products
// of unit u + 1 while it computes dS^T of unit u from the accumulators of the
// previous slot, one score per chunk (its exponential, fma and multiply, and
// half a pack). Each accumulator sums the same products in the same order as
// in bwd_dq_kernel: bit-identical dQ. K/V tiles of 64 keys (two units) in a
// ring of BWD_DQ_SP_RING slots, one LDS array each.
#ifndef BWD_DQ_SP
#define BWD_DQ_SP 1
#endif
// The combined launch takes the pipelined dQ body also when N % 64 is at most
// 32, its empty last unit skipped (RAG 2; identical results): B=16, H=12,
// N=197 17.5-18.9 -> 17.0-17.6 us, B=16, H=16, N=129 17.6-18.7 -> 16.4-17.1
// us, B=32, H=12, N=196 unchanged; the stand-alone dQ kernel at N=196 about
// 5 % faster with the skip.
// Causal rows at d_k = 64 run the dQ kernel with one 32-query block per wave
// (128-query workgroups) at three waves per SIMD: finer blocks balance the
// triangle. Identical results; per launch B=8, H=16, N=4096 399-406 -> 390-392
// us, B=4, H=12, N=2048 65-71 -> 48-49 us, B=4, H=8, N=1024 34 -> 20 us,
// B=16, H=12, N=197 15 -> 10 us.
#ifndef BWD_DQ_CAUSAL_QB1
#define BWD_DQ_CAUSAL_QB1 1
#endif
#ifndef BWD_DQ_SP_RAG2
#define BWD_DQ_SP_RAG2 1
#endif
#ifndef BWD_DQ_SP_RING
#define BWD_DQ_SP_RING 3
#endif
#ifndef BWD_DQ_SP_AHEAD
#define BWD_DQ_SP_AHEAD 2
#endif

template <int WAVES>
struct DqSpShape {
  static constexpr int D = 64, BCK = 64, ROWB = 2 * D, THREADS = 64 * WAVES;
  static constexpr int BR = 32 * WAVES;              // queries per workgroup (32 per wave)
  static constexpr int TILEB = BCK * ROWB;           // one K or V tile (8 KB)
  static constexpr int KDMA = BCK * D / 8 / THREADS; // 16-byte DMAs per lane per tensor per tile
  static_assert(KDMA >= 1 && (BCK * D / 8) % THREADS == 0, "tiles split evenly over the lanes");
  static constexpr int OFF_K = 0, OFF_V = TILEB, SLOTB = 2 * TILEB;
};

// RAG (as dkdv_rag_of): 0 when N is a multiple of the 64-key tile;
// otherwise key rows past N are read as row N - 1 and get probability 0 in
// the last tile, whose second 32-key unit holds keys (RAG 1) or none (RAG 2:
// that unit is not computed).
template <class E, int NS, int WAVES, int RAG>
__device__ __forceinline__ void dq_sp_body(const SpRing& ring, int work, const uint16_t* __restrict__ Q,
                                           const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                           const uint16_t* __restrict__ dO, const float* __restrict__ lse2_in,
                                           const float* __restrict__ ndelta, uint16_t* __restrict__ dQ, int N,
                                           int n_qblk, float c, float scale, int H, Strides sq, Strides sd,
                                           Strides sg) {
  using S = DqSpShape<WAVES>;
  constexpr int D = S::D;
  static_assert(NS == 3 || NS == 4, "ring of 3 or 4 tiles");
  auto slot_base = [&](auto r_) __attribute__((always_inline)) -> unsigned char* {
    constexpr int R = decltype(r_)::value % NS;
    return ring.s[R];
  };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int g = lane >> 4, gi = lane & 15;
  const int dsub = g & 1, er = gi >> 2, qq = gi & 3;
  const int bh = work / n_qblk, qblk = work - bh * n_qblk;
  const size_t hq = head_off(sq, bh, H), hd = head_off(sd, bh, H);
  const size_t hrow = (size_t)bh * N;
  const int q = qblk * S::BR + wave * 32 + l32;  // this lane's query (queries past N compute unused rows)
  const bool ok = q < N;

  // Q and dO fragments of this lane's query (B operands of S^T = K Q^T and
  // dP^T = V dO^T), its lse in log2 units and -delta (as in dq_body).
  u32x4 qf[D / 16], df[D / 16];
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (ok) {
      a = *reinterpret_cast<const u32x4*>(Q + hq + q * sq.n + cc * 16 + h * 8);
      b = *reinterpret_cast<const u32x4*>(dO + hd + q * sd.n + cc * 16 + h * 8);
    }
    qf[cc] = a;
    df[cc] = b;
  }
  const float lse2 = ok ? lse2_in[hrow + q] : 0.f;
  const float dl = ok ? ndelta[hrow + q] : 0.f;

  const Rsrc rK = make_rsrc(K + hq), rV = make_rsrc(V + hq);
  auto dma_tile = [&](int j, auto r_) __attribute__((always_inline)) {
    unsigned char* base = slot_base(r_);
#pragma unroll
    for (int r = 0; r < S::KDMA; ++r) {
      const int slot0 = (wave * S::KDMA + r) * 64;
      const int p = slot0 + lane;
      const int row = p / (D / 8), chunk = (p - row * (D / 8)) ^ swz<S::ROWB>(row);
      const int kr = RAG ? min(j * S::BCK + row, N - 1) : j * S::BCK + row;
      const uint32_t off = (uint32_t)(kr * sq.n + chunk * 8) * 2u;
      dma16(rK, off, base + S::OFF_K + slot0 * 16);
      dma16(rV, off, base + S::OFF_V + slot0 * 16);
    }
  };

  // Per-lane LDS offsets (key block 0 of a tile; the other block and the
  // 16-key halves add whole rows, which leave the swizzle unchanged): K and V
  // rows l32 (chunk 2cc + h), and the transposing K reads of rows 4h + er (+ 8).
  int koff[D / 16], toff[2][2];
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) koff[cc] = tile_off<S::ROWB>(l32, cc * 16 + h * 8);
#pragma unroll
  for (int hi = 0; hi < 2; ++hi)
#pragma unroll
    for (int db = 0; db < 2; ++db) toff[hi][db] = tile_off<S::ROWB>(4 * h + er + 8 * hi, db * 32 + dsub * 16 + 4 * qq);

  // Product m of a slot: m < 4 the dQ^T products of the previous unit (16-key
  // half m >> 1, 32-dim block m & 1: dq_body's order), m >= 4 the S^T and
  // dP^T products of the next unit (b = m - 4: kind b & 1, 16-dim chunk b >> 1).
  auto operand = [&](int m, auto ra_, auto kba_, auto rb_, auto kbb_) __attribute__((always_inline)) -> u32x4 {
    if (m < 4) {
      const unsigned char* T = slot_base(ra_) + S::OFF_K;
      const int rows = (decltype(kba_)::value * 32 + (m >> 1) * 16) * S::ROWB, db = m & 1;
      return cat(lds_read_tr16_b64(T, rows + toff[0][db]), lds_read_tr16_b64(T, rows + toff[1][db]));
    }
    const int b = m - 4;
    const unsigned char* T = slot_base(rb_) + ((b & 1) ? S::OFF_V : S::OFF_K);
    return lds_read_b128(T, decltype(kbb_)::value * 32 * S::ROWB + koff[b >> 1]);
  };

  f32x16 dqacc[2];
#pragma unroll
  for (int db = 0; db < 2; ++db) dqacc[db] = f32x16{};

  // One slot. A (HA): dQ^T += K^T dS^T of the unit in key block KBA of the
  // tile in ring slot RA, from its bf16 dS^T in ya. B (HB): S^T and dP^T -
  // delta of the unit in key block KBB of the tile in slot RB into sn / pn. V
  // (HV): dS^T of the current unit from sv / pv into xd (the pair of entries
  // 2i, 2i + 1 goes to word i & 3 of operand i >> 2).
  // maskV: the current unit (first key kv0) has keys past N, whose P and dS are 0.
  auto slot = [&](auto hasA, auto ra_, auto kba_, const u32x4 (&ya)[2], auto hasB, auto rb_, auto kbb_, f32x16& sn,
                  f32x16& pn, auto hasV, const f32x16& sv, const f32x16& pv, u32x4 (&xd)[2], auto maskV, int kv0)
                  __attribute__((always_inline)) {
    constexpr bool HA = decltype(hasA)::value, HB = decltype(hasB)::value, HV = decltype(hasV)::value;
    constexpr bool MV = decltype(maskV)::value;
    constexpr int AH = BWD_DQ_SP_AHEAD, NO = AH + 1;
    constexpr int M0 = HA ? 0 : 4, M1 = HB ? 12 : 4;  // products [M0, M1)
    u32x4 ops[NO];
    static_for<0, AH>([&](auto a_) __attribute__((always_inline)) {
      constexpr int m = M0 + decltype(a_)::value;
      if constexpr (m < M1) ops[m % NO] = operand(m, ra_, kba_, rb_, kbb_);
    });
    // 12 chunks, one product each (when the slot has all 12); the 16 scores of
    // the current unit are spread over them, score e in chunk 3e / 4.
    float de = 0.f;  // dS of the even entry of the pair
    auto score = [&](auto e_) __attribute__((always_inline)) {
      constexpr int EE = decltype(e_)::value;
      float p = __builtin_amdgcn_exp2f(fmaf(sv[EE], c, -lse2));
      if constexpr (MV) {
        if (kv0 + 8 * (EE >> 2) + 4 * h + (EE & 3) >= N) p = 0.f;
      }
      const float ds = p * (BWD_DQ_DINIT ? pv[EE] : pv[EE] + dl);
      if constexpr (EE & 1) {
        constexpr int i = EE >> 1;
        xd[i >> 2][i & 3] = E::pack(de, ds);
        // An empty use keeps this pair's vector work in this chunk (see BWD_SP_PIN).
        __asm__ volatile("" : : "v"(xd[i >> 2][i & 3]));
      } else {
        de = ds;
      }
    };
    static_for<0, 12>([&](auto k_) __attribute__((always_inline)) {
      constexpr int KK = decltype(k_)::value;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (HB && KK == 0) {
        sn = f32x16{};
#pragma unroll
        for (int e = 0; e < 16; ++e) pn[e] = BWD_DQ_DINIT ? dl : 0.f;
      }
      constexpr int M = M0 + KK;  // this chunk's product (the first M1 - M0 chunks carry one)
      if constexpr (M < M1) {
        if constexpr (M < 4) {
          constexpr int c2 = M >> 1, db = M & 1;
          dqacc[db] = E::mfma(ops[M % NO], ya[c2], dqacc[db]);
        } else {
          constexpr int b = M - 4, cc = b >> 1;
          if constexpr (b & 1)
            pn = E::mfma(ops[M % NO], df[cc], pn);
          else
            sn = E::mfma(ops[M % NO], qf[cc], sn);
        }
        if constexpr (M + AH < M1) ops[(M + AH) % NO] = operand(M + AH, ra_, kba_, rb_, kbb_);
      }
      if constexpr (HV) {
        static_for<(4 * KK + 2) / 3, (4 * KK + 6) / 3>([&](auto e_) __attribute__((always_inline)) { score(e_); });
      }
    });
    __builtin_amdgcn_sched_barrier(0);
  };

  const int nt = (N + S::BCK - 1) / S::BCK;  // tiles (the launcher checks nt >= NS)
  // Before the slot of unit (j, 1): tile j + 1 landed and visible to every
  // wave, every wave done with tile j - 1, whose ring slot takes tile j - 1 + NS.
  auto boundary = [&](int j, auto r_) __attribute__((always_inline)) {
    constexpr int R = decltype(r_)::value;
    if (j + 1 >= nt) return;
    if constexpr (NS == 4) {
      if (j + 2 < nt)
        wait_vmem_below<2 * S::KDMA>();
      else
        wait_vmem_below<0>();
    } else {
      wait_vmem_below<0>();
    }
    __syncthreads();
    if (j - 1 + NS < nt) dma_tile(j - 1 + NS, IntC<(R + NS - 1) % NS>{});
  };

  f32x16 s_0, g_0, s_1, g_1;  // S^T and dP^T - delta of the current units of key blocks 0 and 1
  u32x4 wd_0[2], wd_1[2];     // bf16 dS^T of key blocks 0 and 1
  // Tile j in ring slot R: the slots of units (j, 0) and (j, 1). MASK: the
  // tile holds keys past N (the last tile when ragged).
  auto tile = [&](int j, auto r_, auto first_, auto last_, auto mask_) __attribute__((always_inline)) {
    constexpr int R = decltype(r_)::value;
    constexpr bool FIRST = decltype(first_)::value, LAST = decltype(last_)::value;
    // unit (j, 0): dQ of (j - 1, 1), S / dP of (j, 1), dS of (j, 0)
    slot(BoolC<!FIRST>{}, IntC<(R + NS - 1) % NS>{}, IntC<1>{}, wd_1, BoolC<true>{}, r_, IntC<1>{}, s_1, g_1,
         BoolC<true>{}, s_0, g_0, wd_0, mask_, j * S::BCK);
    boundary(j, r_);
    // unit (j, 1): dQ of (j, 0), S / dP of (j + 1, 0), dS of (j, 1)
    slot(BoolC<true>{}, r_, IntC<0>{}, wd_0, BoolC<!LAST>{}, IntC<(R + 1) % NS>{}, IntC<0>{}, s_0, g_0, BoolC<true>{},
         s_1, g_1, wd_1, mask_, j * S::BCK + 32);
  };

  // Prologue: tiles 0 .. NS - 2 in flight, tile 0 resident, S / dP of unit (0, 0).
  static_for<0, NS - 1>([&](auto r_) __attribute__((always_inline)) { dma_tile(decltype(r_)::value, r_); });
  wait_vmem_below<0>();
  __syncthreads();
  slot(BoolC<false>{}, IntC<0>{}, IntC<0>{}, wd_1, BoolC<true>{}, IntC<0>{}, IntC<0>{}, s_0, g_0, BoolC<false>{}, s_1,
       g_1, wd_0, BoolC<false>{}, 0);
  tile(0, IntC<0>{}, BoolC<true>{}, BoolC<false>{}, BoolC<false>{});
  int j = 1;
  for (; j + NS <= nt - 1; j += NS) {
    static_for<0, NS>([&](auto u_) __attribute__((always_inline)) {
      tile(j + decltype(u_)::value, IntC<(1 + decltype(u_)::value) % NS>{}, BoolC<false>{}, BoolC<false>{},
           BoolC<false>{});
    });
  }
  static_for<0, NS - 1>([&](auto u_) __attribute__((always_inline)) {
    constexpr int U = decltype(u_)::value;
    if (j + U < nt - 1) tile(j + U, IntC<(1 + U) % NS>{}, BoolC<false>{}, BoolC<false>{}, BoolC<false>{});
  });
  // The last tile, nt - 1, in ring slot (nt - 1) % NS (with the key mask when
  // ragged), then dQ of its unit (nt - 1, 1). With RAG 2 that unit has no
  // keys: the tile is the slot of its first unit without the next unit's
  // products, then the dQ products of that first unit.
  static_for<0, NS>([&](auto r_) __attribute__((always_inline)) {
    constexpr int R = decltype(r_)::value;
    if ((nt - 1) % NS == R) {
      if constexpr (RAG == 2) {
        slot(BoolC<true>{}, IntC<(R + NS - 1) % NS>{}, IntC<1>{}, wd_1, BoolC<false>{}, r_, IntC<1>{}, s_1, g_1,
             BoolC<true>{}, s_0, g_0, wd_0, BoolC<true>{}, (nt - 1) * S::BCK);
        slot(BoolC<true>{}, r_, IntC<0>{}, wd_0, BoolC<false>{}, r_, IntC<0>{}, s_0, g_0, BoolC<false>{}, s_1, g_1,
             wd_1, BoolC<false>{}, 0);
      } else {
        tile(nt - 1, r_, BoolC<false>{}, BoolC<true>{}, BoolC<(RAG != 0)>{});
        slot(BoolC<true>{}, r_, IntC<1>{}, wd_1, BoolC<false>{}, r_, IntC<0>{}, s_0, g_0, BoolC<false>{}, s_1, g_1,
             wd_0, BoolC<false>{}, 0);
      }
    }
  });

  // Epilogue: dQ = scale (dQ^T)^T, 16-bit RNE (as dq_body's). Lane: query, dims db*32 + 8jj + 4h + 0..3.
  if (ok) {
    uint16_t* row = dQ + head_off(sg, bh, H) + q * sg.n;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x16& a = dqacc[db];
        const u32x2 w = {E::pack(a[4 * jj] * scale, a[4 * jj + 1] * scale),
                         E::pack(a[4 * jj + 2] * scale, a[4 * jj + 3] * scale)};
        *reinterpret_cast<u32x2*>(row + db * 32 + 8 * jj + 4 * h) = w;
      }
  }
}

template <class E, int NS, int WAVES, int RAG>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_sp_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                      const uint16_t* __restrict__ dO, const float* __restrict__ lse2_in,
                      const float* __restrict__ ndelta, uint16_t* __restrict__ dQ, int N, int n_qblk, int total,
                      float c, float scale, int H, Strides sq, Strides sd, Strides sg) {
  using S = DqSpShape<WAVES>;
  __shared__ __attribute__((aligned(16))) unsigned char ring0[S::SLOTB];
  __shared__ __attribute__((aligned(16))) unsigned char ring1[S::SLOTB];
  __shared__ __attribute__((aligned(16))) unsigned char ring2[S::SLOTB];
  __shared__ __attribute__((aligned(16))) unsigned char ring3[NS == 4 ? S::SLOTB : 16];
  dq_sp_body<E, NS, WAVES, RAG>(SpRing{{ring0, ring1, ring2, ring3}}, xcd_remap(blockIdx.x, total), Q, K, V, dO,
                                   lse2_in, ndelta, dQ, N, n_qblk, c, scale, H, sq, sd, sg);
}

// Work of block `id` of a combined launch without the causal mask: which
// part and which work item. The dK/dV blocks come first (the long ones start
// first and the short dQ blocks fill the tail), each XCD (id % 8) taking its
// eighth of the heads in order; when the heads split evenly over the XCDs,
// each XCD then hands out its dQ blocks in reverse, so that the first of them
// find the heads its last dK/dV blocks read still in its L2. Measured per
// launch (identical results): B=32, H=12, N=196 33.1-35.8 -> 31.7-33.1 us
// (fetched bytes 76 -> 65 MB), B=8, H=16, N=1000 115.7-121.8 -> 115.0-116.9
// us, B=4, H=12, N=2048 162.2-163.2 -> 160.9-161.5 us. Interleaving the parts
// head by head fetched each head once (39.5 MB at N=196) but measured 2-6 %
// slower, since the long dK/dV blocks of the last heads then end the launch.
#ifndef BWD_FUSE_DQ_REVERSE
#define BWD_FUSE_DQ_REVERSE 1
#endif
__device__ __forceinline__ void fused_order(int id, int total1, int total2, int n_kblk, bool& dkdv_part, int& work) {
  dkdv_part = id < total1;
  if (dkdv_part) {
    work = xcd_remap(id, total1);
  } else if (BWD_FUSE_DQ_REVERSE && (total1 / n_kblk) % 8 == 0) {
    const int i2 = id - total1, x = i2 & 7, per = total2 >> 3;
    work = x * per + (per - 1 - (i2 >> 3));
  } else {
    work = xcd_remap(id - total1, total2);
  }
}

// dK/dV and dQ work in one launch (d_k <= 64, where both run two waves per
// SIMD): blocks [0, total1) are dK/dV workgroups, the rest dQ workgroups, so
// dQ work fills the CUs that the last dK/dV workgroups leave idle instead of
// waiting for a second launch. total1 is a multiple of 8, so both halves keep
// their XCD assignment.
// Launch shape of the fused kernel: one 32-query block per dQ wave (128
// queries per dQ workgroup), and 32-query dK/dV steps for rows shorter than
// BWD_FUSE_MB1_N (64-query steps otherwise). Measured per launch (identical
// outputs): B=32, H=12, N=196 45.9 -> 38.5 us; causal B=16, H=12, N=197
// 22.8 -> 18.6 us; B=4, H=12, N=2048 190.4 -> 182.7 us (32-query dK/dV steps
// there: 192.4 us). Three waves per SIMD spill (168 registers) and measured
// 1.3-2x slower.
#ifndef BWD_FUSE_QB
#define BWD_FUSE_QB 1
#endif
#ifndef BWD_FUSE_MB1_N
#define BWD_FUSE_MB1_N 1024
#endif
#ifndef BWD_FUSE_WPE
#define BWD_FUSE_WPE BWD_WAVES_PER_EU
#endif
// The combined launch takes the pipelined dK/dV body where that kernel applies.
// Measured per launch (bit-identical outputs): B=32, H=12, N=196 38.5 / 36.1
// -> 35.0 / 34.0 us (two runs), B=8, H=16, N=1000 141 -> 122 us, B=4, H=12,
// N=2048 178 -> 172 us; the pipelined stand-alone dK/dV kernel on ragged rows
// 28 -> 23.6 us at N=196 and 95 -> 70 us at N=1000.
#ifndef BWD_SP_FUSE
#define BWD_SP_FUSE 1
#endif
template <class E, int D, int MB, int QB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(BWD_FUSE_WPE, BWD_FUSE_WPE)))
void bwd_dkdv_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                        const uint16_t* __restrict__ dO, const float* __restrict__ lse2, const float* __restrict__ ndelta,
                        uint16_t* __restrict__ dQ, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N,
                        int n_kblk, int total1, int n_qblk, int total2, float c, float scale,
                        const int* __restrict__ kv_len, int H, int causal, Strides sq, Strides sd, Strides sg) {
  constexpr int L1 = DkdvShape<D, MB>::LDSB, L2 = DqShape<D, QB>::BUFB;
  __shared__ __attribute__((aligned(16))) unsigned char smem[L1 > L2 ? L1 : L2];
  __shared__ __attribute__((aligned(16))) unsigned char smem1[L2];
  // Under the causal mask the bodies order their blocks heaviest first from
  // the plain per-part XCD ranges.
  bool dkdv_part = blockIdx.x < total1;
  int work = dkdv_part ? xcd_remap(blockIdx.x, total1) : xcd_remap(blockIdx.x - total1, total2);
  if (!causal) fused_order(blockIdx.x, total1, total2, n_kblk, dkdv_part, work);
  if (dkdv_part)
    dkdv_body<E, D, MB, 1>(smem, work, Q, K, V, dO, lse2, ndelta, dK, dV, N, n_kblk, total1, c, scale, kv_len, H, causal,
                           sq, sd, sg);
  else
    dq_body<E, D, QB>(smem, smem1, work, Q, K, V, dO, lse2, ndelta, dQ, N, n_qblk, total2, c, scale, kv_len, H, causal,
                      sq, sd, sg);
}

// The combined launch with the pipelined dK/dV body (d_k = 64, no mask, at
// least BWD_SP_RING 64-row steps; a ragged last step is masked): blocks [0,
// total1) run dkdv_sp_body on 128 keys each, the rest dQ on 128 queries each,
// with the pipelined dq_sp_body where its 64-key tiles cover no more keys
// than dq_body's 32-key steps (DQSP: N % 64 is 0 or above 32), dq_body
// otherwise, on the same ring of LDS arrays. Measured per launch (identical
// results): B=4, H=12, N=2048 173-176 -> 167 us and B=8, H=16, N=1000 123-128
// -> 119 us with dq_sp_body; at B=32, H=12, N=196 (256 keys in tiles against
// 224 in steps) it measured 3 % slower than with dq_body.
template <class E, int NS, int RAG, bool DQSP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_sp_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                           const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                           const float* __restrict__ lse2, const float* __restrict__ ndelta, uint16_t* __restrict__ dQ,
                           uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N, int n_kblk, int total1,
                           int n_qblk, int total2, float c, float scale, const int* __restrict__ kv_len, int H,
                           int causal, Strides sq, Strides sd, Strides sg) {
  using S = DkdvSpShape<kThreads / 64>;
  static_assert(DqSpShape<kThreads / 64>::SLOTB <= S::SLOTB && DqShape<S::D, 1>::BUFB <= S::SLOTB,
                "a dQ tile or step buffer fits in a ring slot");
  __shared__ __attribute__((aligned(16))) unsigned char ring0[S::SLOTB];
  __shared__ __attribute__((aligned(16))) unsigned char ring1[S::SLOTB];
  __shared__ __attribute__((aligned(16))) unsigned char ring2[S::SLOTB];
  __shared__ __attribute__((aligned(16))) unsigned char ring3[NS == 4 ? S::SLOTB : 16];
  bool dkdv_part;
  int work;
  fused_order(blockIdx.x, total1, total2, n_kblk, dkdv_part, work);
  if (dkdv_part)
    dkdv_sp_body<E, NS, kThreads / 64, RAG, false>(SpRing{{ring0, ring1, ring2, ring3}}, work, Q, K, V, dO, lse2,
                                                   ndelta, dK, dV, N, n_kblk, total1, c, scale, H, sq, sd, sg);
  else if constexpr (DQSP)
    dq_sp_body<E, NS, kThreads / 64, RAG>(SpRing{{ring0, ring1, ring2, ring3}}, work, Q, K, V, dO, lse2, ndelta,
                                                 dQ, N, n_qblk, c, scale, H, sq, sd, sg);
  else
    dq_body<E, S::D, 1>(ring0, ring1, work, Q, K, V, dO, lse2, ndelta, dQ, N, n_qblk, total2, c, scale, kv_len, H,
                        causal, sq, sd, sg);
}

// ---------------------------------------------------------------- fp32 backward
// fp32 storage and fp32 arithmetic throughout (vector ALU), the same three
// deterministic stages. LP lanes share a row (a key in stage 1, a query in
// stage 2): lane part p owns columns [p * D/LP, (p+1) * D/LP) of that row, dot
// products are split over the LP lanes and summed with xor shuffles. LP = 4
// (64 rows per workgroup) where the grid is large; LP = 16 (16 rows per
// workgroup, four times the workgroups) for few heads and short sequences at
// D >= 64, where 64-row workgroups would leave most CUs idle.
constexpr int kF32Step = 32;   // rows of the other side staged in LDS per step

__global__ __launch_bounds__(256) void bwd_prep_f32_kernel(const float* __restrict__ O, const float* __restrict__ dO,
                                                           const float* __restrict__ LSE, float* __restrict__ lse_out,
                                                           float* __restrict__ ndelta, long rows, int D) {
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = gid >> 3;
  const int part = (int)(gid & 7);
  float s = 0.f;
  if (row < rows)
    for (int c = part; c < D; c += 8) s = fmaf(O[row * D + c], dO[row * D + c], s);
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 4);
  if (row < rows && part == 0) {
    ndelta[row] = -s;
    lse_out[row] = LSE[row];
  }
}

template <int LP>
__device__ __forceinline__ float sum_lanes(float x) {
#pragma unroll
  for (int o = 1; o < LP; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

// Stage 1: dV_j = sum_i P_ij dO_i, dK_j = scale * sum_i dS_ij Q_i for 256 / LP keys j.
template <int D, int LP>
__global__ __launch_bounds__(256) void bwd_dkdv_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                           const float* __restrict__ V, const float* __restrict__ dO,
                                                           const float* __restrict__ LSE, const float* __restrict__ ndelta,
                                                           float* __restrict__ dK, float* __restrict__ dV, int N,
                                                           int n_kblk, float scale) {
  constexpr int DC = D / LP;
  __shared__ float Qs[kF32Step][D], dOs[kF32Step][D], Ls[kF32Step], Ds[kF32Step];
  const int tid = threadIdx.x, part = tid % LP;
  const int bh = blockIdx.x / n_kblk, kblk = blockIdx.x - bh * n_kblk;
  const size_t head = (size_t)bh * N * D;
  const int key = kblk * (256 / LP) + tid / LP;
  const bool ok = key < N;
  float kr[DC], vr[DC], dk[DC], dv[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    kr[c] = ok ? K[head + (size_t)key * D + part * DC + c] : 0.f;
    vr[c] = ok ? V[head + (size_t)key * D + part * DC + c] : 0.f;
    dk[c] = 0.f;
    dv[c] = 0.f;
  }
  for (int i0 = 0; i0 < N; i0 += kF32Step) {
    __syncthreads();
    for (int idx = tid; idx < kF32Step * D; idx += 256) {
      const int r = idx / D, c = idx - r * D;
      const bool in = i0 + r < N;
      Qs[r][c] = in ? Q[head + (size_t)(i0 + r) * D + c] : 0.f;
      dOs[r][c] = in ? dO[head + (size_t)(i0 + r) * D + c] : 0.f;
    }
    if (tid < kF32Step) {
      const bool in = i0 + tid < N;
      Ls[tid] = in ? LSE[(size_t)bh * N + i0 + tid] : 0.f;
      Ds[tid] = in ? ndelta[(size_t)bh * N + i0 + tid] : 0.f;
    }
    __syncthreads();
    const int rows = min(kF32Step, N - i0);
    for (int r = 0; r < rows; ++r) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        s = fmaf(Qs[r][part * DC + c], kr[c], s);
        dp = fmaf(dOs[r][part * DC + c], vr[c], dp);
      }
      s = sum_lanes<LP>(s);
      dp = sum_lanes<LP>(dp);
      const float p = ok ? expf(s * scale - Ls[r]) : 0.f;
      const float ds = p * (dp + Ds[r]);
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        dv[c] = fmaf(p, dOs[r][part * DC + c], dv[c]);
        dk[c] = fmaf(ds, Qs[r][part * DC + c], dk[c]);
      }
    }
  }
  if (ok) {
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      dV[head + (size_t)key * D + part * DC + c] = dv[c];
      dK[head + (size_t)key * D + part * DC + c] = dk[c] * scale;
    }
  }
}

// Stage 2: dQ_i = scale * sum_j dS_ij K_j for 256 / LP queries i.
template <int D, int LP>
__global__ __launch_bounds__(256) void bwd_dq_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                         const float* __restrict__ V, const float* __restrict__ dO,
                                                         const float* __restrict__ LSE, const float* __restrict__ ndelta,
                                                         float* __restrict__ dQ, int N, int n_qblk, float scale) {
  constexpr int DC = D / LP;
  __shared__ float Ks[kF32Step][D], Vs[kF32Step][D];
  const int tid = threadIdx.x, part = tid % LP;
  const int bh = blockIdx.x / n_qblk, qblk = blockIdx.x - bh * n_qblk;
  const size_t head = (size_t)bh * N * D;
  const int q = qblk * (256 / LP) + tid / LP;
  const bool ok = q < N;
  float qr[DC], dor[DC], dq[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    qr[c] = ok ? Q[head + (size_t)q * D + part * DC + c] : 0.f;
    dor[c] = ok ? dO[head + (size_t)q * D + part * DC + c] : 0.f;
    dq[c] = 0.f;
  }
  const float l = ok ? LSE[(size_t)bh * N + q] : 0.f;
  const float nd = ok ? ndelta[(size_t)bh * N + q] : 0.f;
  for (int j0 = 0; j0 < N; j0 += kF32Step) {
    __syncthreads();
    for (int idx = tid; idx < kF32Step * D; idx += 256) {
      const int r = idx / D, c = idx - r * D;
      const bool in = j0 + r < N;
      Ks[r][c] = in ? K[head + (size_t)(j0 + r) * D + c] : 0.f;
      Vs[r][c] = in ? V[head + (size_t)(j0 + r) * D + c] : 0.f;
    }
    __syncthreads();
    const int rows = min(kF32Step, N - j0);
    for (int r = 0; r < rows; ++r) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        s = fmaf(qr[c], Ks[r][part * DC + c], s);
        dp = fmaf(dor[c], Vs[r][part * DC + c], dp);
      }
      s = sum_lanes<LP>(s);
      dp = sum_lanes<LP>(dp);
      const float p = ok ? expf(s * scale - l) : 0.f;
      const float ds = p * (dp + nd);
#pragma unroll
      for (int c = 0; c < DC; ++c) dq[c] = fmaf(ds, Ks[r][part * DC + c], dq[c]);
    }
  }
  if (ok) {
#pragma unroll
    for (int c = 0; c < DC; ++c) dQ[head + (size_t)q * D + part * DC + c] = dq[c] * scale;
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// Stages 1 and 2 run as one launch when both kernels run two waves per SIMD
// with the same launch shape (d_k <= 64, one key block per wave), the dK/dV
// grid is a multiple of the 8 XCDs, and it is small enough (at most 4
// workgroups per CU) for the tail of the dK/dV launch to matter: measured per
// step, 70 -> 64 us at B=32, H=12, N=196 and 277 -> 268 us at B=4, H=12,
// N=2048. Against the two launches (the dK/dV one pipelined where the rows
// allow), per backward: 768 dK/dV workgroups 108 -> 99 us, 1024 246 -> 239
// us, but 1536 336 -> 350 us and 2048 1648 -> 1761 us.
bool bwd_can_fuse(int B, int H, int N, int d) {
#if BWD_FUSE
  if (d > 64 || BWD_KBW64 != 1 || BWD_MB64 != 2) return false;
  const long total1 = (long)((N + 127) / 128) * B * H;
  return total1 % 8 == 0 && total1 <= 4 * 256;
#else
  (void)B, (void)H, (void)N, (void)d;
  return false;
#endif
}

// The stand-alone dQ launch takes the pipelined kernel (one 32-query block per
// wave) where rows are unmasked, at least BWD_DQ_SP_RING 64-key tiles long at
// d_k = 64, and the grid of the single-phase kernel (two blocks per wave, 256
// queries per workgroup) would be under 4 workgroups per CU: measured per
// launch (identical dQ) B=4, H=12, N=2048 87-97 -> 74 us, B=8, H=16, N=1024
// 56-62 -> 52 us, B=2, H=3, N=192 9.6 -> 6.5 us, but B=8, H=16, N=4096 (2048
// workgroups) 687 -> 702 us and B=2, H=16, N=8192 697 -> 720 us: with ample
// workgroups the two-block kernel's operand reuse (each K / V fragment feeds
// two products) wins.
static bool bwd_dq_pipelined(int B, int H, int N, int d, int causal, bool kv_len) {
  if (!BWD_DQ_SP || d != 64 || causal || kv_len || (N + 63) / 64 < BWD_DQ_SP_RING) return false;
  return (long)B * H * ((N + 255) / 256) < 4 * 256;
}

// Workspace: lse * log2(e), then -delta; fp32 [B*H*N] each, 256-byte aligned.
size_t bwd_workspace_bytes(int B, int H, int N, int d) {
  (void)d;
  return 2 * align256((size_t)B * H * N * 4);
}

template <class E, int D>
static hipError_t launch_bwd_stage_t(int stage, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     const uint16_t* o, const float* lse, const uint16_t* dO, uint16_t* dq,
                                     uint16_t* dk, uint16_t* dv, int B, int H, int N, float scale, int causal,
                                     const int* kv_len, const Strides* st, void* workspace, hipStream_t stream) {
  const long rows = (long)B * H * N;
  float* lse2 = reinterpret_cast<float*>(workspace);
  float* ndelta = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(workspace) + align256(rows * 4));
  const float c = scale * kLog2e;
  if (stage == 0) {
    hipLaunchKernelGGL((bwd_prep_kernel<E, D>), dim3((unsigned)((rows * 8 + 255) / 256)), dim3(256), 0, stream, o, dO,
                       lse, lse2, ndelta, rows, N, H, st[1], st[2]);
  } else if (stage == 3) {  // stages 1 and 2 in one launch (callers check bwd_can_fuse)
    if constexpr (D <= 64) {  // only instantiated where bwd_can_fuse can say yes
      constexpr int QB = BWD_FUSE_QB;
      constexpr int BCK = 4 * 32;
      const int n_kblk = (N + BCK - 1) / BCK, total1 = n_kblk * B * H;
      constexpr int BR = DqShape<D, QB>::BR;
      const int n_qblk = (N + BR - 1) / BR, total2 = n_qblk * B * H;
      if (D == 64 && BWD_SP_FUSE && BWD_SP && !causal && !kv_len && (N + 63) / 64 >= BWD_SP_RING) {
        static_assert(DqSpShape<kThreads / 64>::BR == BR && QB == 1, "the same dQ grid for both dQ bodies");
        const dim3 grid(total1 + total2);
#define ATTN_SP_DQ(RAG, DQSP)                                                                                      \
  hipLaunchKernelGGL((bwd_dkdv_sp_dq_kernel<E, BWD_SP_RING, RAG, DQSP>), grid, dim3(kThreads), 0, stream, q, k, v, dO, \
                     lse2, ndelta, dq, dk, dv, N, n_kblk, total1, n_qblk, total2, c, scale, kv_len, H, causal, st[0], \
                     st[2], st[3])
        // dq_sp_body where N % 64 is 0 or above 32 (dkdv_rag_of(N) 0 or 1).
        switch (dkdv_rag_of(N)) {
#if BWD_DQ_SP
          case 0: ATTN_SP_DQ(0, true); break;
          case 1: ATTN_SP_DQ(1, true); break;
#else
          case 0: ATTN_SP_DQ(0, false); break;
          case 1: ATTN_SP_DQ(1, false); break;
#endif
          default:
            if (BWD_DQ_SP && BWD_DQ_SP_RAG2)
              ATTN_SP_DQ(2, true);
            else
              ATTN_SP_DQ(2, false);
            break;
        }
#undef ATTN_SP_DQ
      } else if (D == 64 && N < BWD_FUSE_MB1_N)  // 32-query steps split evenly over the DMA lanes at d_k = 64 only
        hipLaunchKernelGGL((bwd_dkdv_dq_kernel<E, D, (D == 64 ? 1 : 2), QB>), dim3(total1 + total2), dim3(kThreads),
                           0, stream, q, k, v, dO, lse2, ndelta, dq, dk, dv, N, n_kblk, total1, n_qblk, total2, c,
                           scale, kv_len, H, causal, st[0], st[2], st[3]);
      else
        hipLaunchKernelGGL((bwd_dkdv_dq_kernel<E, D, 2, QB>), dim3(total1 + total2), dim3(kThreads), 0, stream, q, k,
                           v, dO, lse2, ndelta, dq, dk, dv, N, n_kblk, total1, n_qblk, total2, c, scale, kv_len, H,
                           causal, st[0], st[2], st[3]);
    } else {
      return hipErrorInvalidValue;
    }
  } else if (stage == 1) {
    if constexpr (D == 64) {
      constexpr int NS = BWD_SP_RING;
      // Causal rows of whole 128-key blocks (BWD_SP_CAUSAL) too: every block then has at least two steps.
      const bool sp_causal = causal && BWD_SP_CAUSAL && N % 128 == 0;
      if (BWD_SP && (!causal || sp_causal) && !kv_len && (N + 63) / 64 >= NS) {
        constexpr int W = BWD_SP_WAVES, BCK = DkdvSpShape<W>::BCK;
        const int n_kblk = (N + BCK - 1) / BCK, total = n_kblk * B * H;
#define ATTN_SP_DKDV(RAG, CAUSAL)                                                                            \
  hipLaunchKernelGGL((bwd_dkdv_sp_kernel<E, NS, W, RAG, CAUSAL>), dim3(total), dim3(64 * W), 0, stream, q, k, v, dO, \
                     lse2, ndelta, dk, dv, N, n_kblk, total, c, scale, H, st[0], st[2], st[3])
        if (sp_causal) {
          ATTN_SP_DKDV(0, true);
        } else {
          switch (dkdv_rag_of(N)) {
            case 0: ATTN_SP_DKDV(0, false); break;
            case 1: ATTN_SP_DKDV(1, false); break;
            default: ATTN_SP_DKDV(2, false); break;
          }
        }
#undef ATTN_SP_DKDV
        return hipGetLastError();
      }
    }
    constexpr int MB = D == 64 ? BWD_MB64 : 2, KBW = D == 64 ? BWD_KBW64 : 1;
    constexpr int BCK = 4 * 32 * KBW;
    const int n_kblk = (N + BCK - 1) / BCK;
    const int total = n_kblk * B * H;
    hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, MB, KBW>), dim3(total), dim3(kThreads), 0, stream, q, k, v, dO, lse2, ndelta,
                       dk, dv, N, n_kblk, total, c, scale, kv_len, H, causal, st[0], st[2], st[3]);
  } else {
    if constexpr (D == 64) {
      constexpr int NS = BWD_DQ_SP_RING;
      if (bwd_dq_pipelined(B, H, N, D, causal, kv_len != nullptr)) {
        constexpr int W = 4, BR = DqSpShape<W>::BR;
        const int n_qblk = (N + BR - 1) / BR, total = n_qblk * B * H;
#define ATTN_SP_DQ1(RAG)                                                                                     \
  hipLaunchKernelGGL((bwd_dq_sp_kernel<E, NS, W, RAG>), dim3(total), dim3(64 * W), 0, stream, q, k, v, dO, lse2,  \
                     ndelta, dq, N, n_qblk, total, c, scale, H, st[0], st[2], st[3])
        switch (dkdv_rag_of(N)) {
          case 0: ATTN_SP_DQ1(0); break;
          case 1: ATTN_SP_DQ1(1); break;
          default: ATTN_SP_DQ1(2); break;
        }
#undef ATTN_SP_DQ1
        return hipGetLastError();
      }
    }
    if constexpr (D == 64) {
      if (causal && BWD_DQ_CAUSAL_QB1) {  // 128-query workgroups, three waves per SIMD
        constexpr int BR = DqShape<D, 1>::BR;
        const int n_qblk = (N + BR - 1) / BR;
        const int total = n_qblk * B * H;
        hipLaunchKernelGGL((bwd_dq_kernel<E, D, 1>), dim3(total), dim3(kThreads), 0, stream, q, k, v, dO, lse2, ndelta,
                           dq, N, n_qblk, total, c, scale, kv_len, H, causal, st[0], st[2], st[3]);
        return hipGetLastError();
      }
    }
    constexpr int QB = D <= 64 ? BWD_DQ_QB64 : 1;
    constexpr int BR = DqShape<D, QB>::BR;
    const int n_qblk = (N + BR - 1) / BR;
    const int total = n_qblk * B * H;
    hipLaunchKernelGGL((bwd_dq_kernel<E, D, QB>), dim3(total), dim3(kThreads), 0, stream, q, k, v, dO, lse2, ndelta, dq,
                       N, n_qblk, total, c, scale, kv_len, H, causal, st[0], st[2], st[3]);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_16_stage(bool f16, int stage, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const uint16_t* o, const float* lse, const uint16_t* dO, uint16_t* dq, uint16_t* dk,
                                 uint16_t* dv, int B, int H, int N, int d, float scale, int causal,
                                 const int* kv_len, const Strides* st, void* workspace,
                               hipStream_t stream) {
#define ATTN_BWD_STAGE(E, D) \
  launch_bwd_stage_t<E, D>(stage, q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, causal, kv_len, st, workspace, \
                           stream)
  if (f16) {
    switch (d) {
      case 32: return ATTN_BWD_STAGE(F16, 32);
      case 64: return ATTN_BWD_STAGE(F16, 64);
      case 96: return ATTN_BWD_STAGE(F16, 96);
      default: return ATTN_BWD_STAGE(F16, 128);
    }
  }
  switch (d) {
    case 32: return ATTN_BWD_STAGE(Bf16, 32);
    case 64: return ATTN_BWD_STAGE(Bf16, 64);
    case 96: return ATTN_BWD_STAGE(Bf16, 96);
    default: return ATTN_BWD_STAGE(Bf16, 128);
  }
#undef ATTN_BWD_STAGE
}

template <int D, int LP>
static void launch_f32_stage_lp(int stage, int BH, const float* q, const float* k, const float* v, const float* dO,
                                const float* lse_ws, const float* ndelta, float* dq, float* dk, float* dv, int N,
                                float scale, hipStream_t stream) {
  const int nblk = (N + 256 / LP - 1) / (256 / LP);
  const dim3 grid((unsigned)(nblk * BH));
  if (stage == 1)
    hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D, LP>), grid, dim3(256), 0, stream, q, k, v, dO, lse_ws, ndelta, dk, dv,
                       N, nblk, scale);
  else
    hipLaunchKernelGGL((bwd_dq_f32_kernel<D, LP>), grid, dim3(256), 0, stream, q, k, v, dO, lse_ws, ndelta, dq, N,
                       nblk, scale);
}

// 16 lanes per row while the 64-row grid would be under 1024 workgroups (four
// per CU), for D >= 64. At D = 32 a lane would keep 2 columns and the 16-lane
// sums cost more than the extra workgroups gain (measured 8-18 % slower).
template <int D>
static void launch_f32_stage_t(int stage, int B, int H, const float* q, const float* k, const float* v,
                               const float* dO, const float* lse_ws, const float* ndelta, float* dq, float* dk,
                               float* dv, int N, float scale, hipStream_t stream) {
  if (D >= 64 && (long)B * H * ((N + 63) / 64) < 1024)
    launch_f32_stage_lp<D, (D >= 64 ? 16 : 4)>(stage, B * H, q, k, v, dO, lse_ws, ndelta, dq, dk, dv, N, scale,
                                               stream);
  else
    launch_f32_stage_lp<D, 4>(stage, B * H, q, k, v, dO, lse_ws, ndelta, dq, dk, dv, N, scale, stream);
}

hipError_t launch_bwd_f32_stage(int stage, const float* q, const float* k, const float* v, const float* o,
                                const float* lse, const float* dO, float* dq, float* dk, float* dv, int B, int H, int N,
                                int d, float scale, void* workspace, hipStream_t stream) {
  const long rows = (long)B * H * N;
  float* lse_ws = reinterpret_cast<float*>(workspace);
  float* ndelta = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(workspace) + align256(rows * 4));
  if (stage == 0) {
    hipLaunchKernelGGL(bwd_prep_f32_kernel, dim3((unsigned)((rows * 8 + 255) / 256)), dim3(256), 0, stream, o, dO,
                       lse, lse_ws, ndelta, rows, d);
    return hipGetLastError();
  }
  switch (d) {
    case 32: launch_f32_stage_t<32>(stage, B, H, q, k, v, dO, lse_ws, ndelta, dq, dk, dv, N, scale, stream); break;
    case 64: launch_f32_stage_t<64>(stage, B, H, q, k, v, dO, lse_ws, ndelta, dq, dk, dv, N, scale, stream); break;
    case 96: launch_f32_stage_t<96>(stage, B, H, q, k, v, dO, lse_ws, ndelta, dq, dk, dv, N, scale, stream); break;
    default: launch_f32_stage_t<128>(stage, B, H, q, k, v, dO, lse_ws, ndelta, dq, dk, dv, N, scale, stream);
  }
  return hipGetLastError();
}

}  // namespace attn
