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

    // ---- S^T = K Q^T and dP^T = V dO^T: 32 keys x (32*QB) queries.
    f32x16 sacc[QB], pacc[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      sacc[qb] = f32x16{};
      pacc[qb] = f32x16{};
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
        dsb[qb][e >> 3][(e >> 1) & 3] = E::pack(p0 * (pacc[qb][e] + dl[qb]), p1 * (pacc[qb][e + 1] + dl[qb]));
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

template <class E, int D, int QB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(BWD_WAVES_PER_EU, BWD_WAVES_PER_EU)))
void bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                   const uint16_t* __restrict__ dO, const float* __restrict__ lse2_in, const float* __restrict__ ndelta,
                   uint16_t* __restrict__ dQ, int N, int n_qblk, int total, float c, float scale,
                   const int* __restrict__ kv_len, int H, int causal, Strides sq, Strides sd, Strides sg) {
  __shared__ __attribute__((aligned(16))) unsigned char buf0[DqShape<D, QB>::BUFB];
  __shared__ __attribute__((aligned(16))) unsigned char buf1[DqShape<D, QB>::BUFB];
  dq_body<E, D, QB>(buf0, buf1, xcd_remap(blockIdx.x, total), Q, K, V, dO, lse2_in, ndelta, dQ, N, n_qblk, total, c, scale,
                    kv_len, H, causal, sq, sd, sg);
}

// dK/dV and dQ work in one launch (d_k <= 64, where both run two waves per
// SIMD): blocks [0, total1) are dK/dV workgroups, the rest dQ workgroups, so
// dQ work fills the CUs that the last dK/dV workgroups leave idle instead of
// waiting for a second launch. total1 is a multiple of 8, so both halves keep
// their XCD assignment.
template <class E, int D, int MB, int QB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(BWD_WAVES_PER_EU, BWD_WAVES_PER_EU)))
void bwd_dkdv_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                        const uint16_t* __restrict__ dO, const float* __restrict__ lse2, const float* __restrict__ ndelta,
                        uint16_t* __restrict__ dQ, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N,
                        int n_kblk, int total1, int n_qblk, int total2, float c, float scale,
                        const int* __restrict__ kv_len, int H, int causal, Strides sq, Strides sd, Strides sg) {
  constexpr int L1 = DkdvShape<D, MB>::LDSB, L2 = DqShape<D, QB>::BUFB;
  __shared__ __attribute__((aligned(16))) unsigned char smem[L1 > L2 ? L1 : L2];
  __shared__ __attribute__((aligned(16))) unsigned char smem1[L2];
  const int id = blockIdx.x;
  if (id < total1)
    dkdv_body<E, D, MB, 1>(smem, xcd_remap(id, total1), Q, K, V, dO, lse2, ndelta, dK, dV, N, n_kblk, total1, c, scale,
                           kv_len, H, causal, sq, sd, sg);
  else
    dq_body<E, D, QB>(smem, smem1, xcd_remap(id - total1, total2), Q, K, V, dO, lse2, ndelta, dQ, N, n_qblk, total2, c, scale,
                      kv_len, H, causal, sq, sd, sg);
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
// grid is a multiple of the 8 XCDs, and it is small enough (at most 8
// workgroups per CU) for the tail of the dK/dV launch to matter: measured per
// step, 70 -> 64 us at B=32, H=12, N=196 and 277 -> 268 us at B=4, H=12,
// N=2048, but no change at B=8, H=16, N=4096 (4096 dK/dV workgroups).
bool bwd_can_fuse(int B, int H, int N, int d) {
#if BWD_FUSE
  if (d > 64 || BWD_KBW64 != 1 || BWD_MB64 != 2) return false;
  const long total1 = (long)((N + 127) / 128) * B * H;
  return total1 % 8 == 0 && total1 <= 8 * 256;
#else
  (void)B, (void)H, (void)N, (void)d;
  return false;
#endif
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
      constexpr int QB = 2;
      constexpr int BCK = 4 * 32;
      const int n_kblk = (N + BCK - 1) / BCK, total1 = n_kblk * B * H;
      constexpr int BR = DqShape<D, QB>::BR;
      const int n_qblk = (N + BR - 1) / BR, total2 = n_qblk * B * H;
      hipLaunchKernelGGL((bwd_dkdv_dq_kernel<E, D, 2, QB>), dim3(total1 + total2), dim3(kThreads), 0, stream, q, k,
                         v, dO, lse2, ndelta, dq, dk, dv, N, n_kblk, total1, n_qblk, total2, c, scale, kv_len, H,
                         causal, st[0], st[2], st[3]);
    } else {
      return hipErrorInvalidValue;
    }
  } else if (stage == 1) {
    constexpr int MB = D == 64 ? BWD_MB64 : 2, KBW = D == 64 ? BWD_KBW64 : 1;
    constexpr int BCK = 4 * 32 * KBW;
    const int n_kblk = (N + BCK - 1) / BCK;
    const int total = n_kblk * B * H;
    hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, MB, KBW>), dim3(total), dim3(kThreads), 0, stream, q, k, v, dO, lse2, ndelta,
                       dk, dv, N, n_kblk, total, c, scale, kv_len, H, causal, st[0], st[2], st[3]);
  } else {
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
