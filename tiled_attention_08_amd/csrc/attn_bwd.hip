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
// Three launches on one stream:
//   1. bwd_prep_kernel    delta = rowsum(dO * O) (fp32), zero the fp32 dQ accumulator;
//   2. bwd_main_kernel    one workgroup per (head, block of 128 keys); loops over
//                         64-query steps, recomputes S and P, accumulates dK and dV
//                         in registers and adds each step's dQ share into the
//                         fp32 accumulator with float atomics;
//   3. bwd_dq_kernel      dQ = bf16(scale * accumulator).
// In the main kernel a key is a lane column (S = Q K^T, m = query, n = key),
// so dV^T = dO^T P and dK^T = Q^T dS take P and dS straight from registers;
// dO^T and Q^T come from transposing LDS reads of the row-major tiles. dQ
// needs dS with the key as contraction index, so dS makes one round trip
// through LDS (written as [key][query], read back transposed) and dQ = dS K
// is accumulated with queries as accumulator rows.
#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {

namespace {

constexpr int kThreads = 256;
constexpr int BCK = kBwdKeysPerBlock;    // keys per workgroup (32 per wave)
constexpr int BRQ = kBwdQueriesPerStep;  // queries per step

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---------------------------------------------------------------- 1. prep
// 8 lanes per row; each lane covers D/8 consecutive elements.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
                                                       float* __restrict__ delta, float* __restrict__ dq_acc,
                                                       long rows) {
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = gid >> 3;
  const int part = (int)(gid & 7);
  constexpr int PER = D / 8;  // elements per lane
  float s = 0.f;
  if (row < rows) {
    const uint16_t* o = O + row * D + part * PER;
    const uint16_t* g = dO + row * D + part * PER;
#pragma unroll
    for (int c = 0; c < PER; c += 8) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(o + c);
      const u32x4 b = *reinterpret_cast<const u32x4*>(g + c);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        s = fmaf(__uint_as_float(a[w] << 16), __uint_as_float(b[w] << 16), s);
        s = fmaf(__uint_as_float(a[w] & 0xffff0000u), __uint_as_float(b[w] & 0xffff0000u), s);
      }
    }
    float* z = dq_acc + row * D + part * PER;
#pragma unroll
    for (int c = 0; c < PER; c += 4) *reinterpret_cast<float4*>(z + c) = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 4);
  if (row < rows && part == 0) delta[row] = s;
}

// ---------------------------------------------------------------- 3. dq convert
__global__ __launch_bounds__(256) void bwd_dq_kernel(const float* __restrict__ acc, uint16_t* __restrict__ dq,
                                                     long n8, float scale) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const float4 a = reinterpret_cast<const float4*>(acc)[2 * i];
  const float4 b = reinterpret_cast<const float4*>(acc)[2 * i + 1];
  const u32x4 w = {pack_bf16(a.x * scale, a.y * scale), pack_bf16(a.z * scale, a.w * scale),
                   pack_bf16(b.x * scale, b.y * scale), pack_bf16(b.z * scale, b.w * scale)};
  reinterpret_cast<u32x4*>(dq)[i] = w;
}

// ---------------------------------------------------------------- 2. main
template <int D>
struct BwdShape {
  static constexpr int ROWB = D * 2;
  static constexpr int KTILEB = BCK * ROWB;             // resident K block
  static constexpr int QTILEB = BRQ * ROWB;             // one Q or dO step tile
  static constexpr int DSROWB = BRQ * 2;                // dS^T row: 64 queries
  static constexpr int DSB = BCK * DSROWB;              // dS^T tile
  static constexpr int KCPT = BCK * D / 8 / kThreads;   // 16-byte chunks per thread, K block
  static constexpr int QCPT = BRQ * D / 8 / kThreads;   // 16-byte chunks per thread, Q/dO tile
  static constexpr int OFF_K = 0;
  static constexpr int OFF_Q = OFF_K + KTILEB;
  static constexpr int OFF_DO = OFF_Q + 2 * QTILEB;
  static constexpr int OFF_L = OFF_DO + 2 * QTILEB;     // lse * log2(e), two buffers
  static constexpr int OFF_DL = OFF_L + 2 * BRQ * 4;    // delta, two buffers
  static constexpr int OFF_DS = OFF_DL + 2 * BRQ * 4;
  static constexpr int LDSB = OFF_DS + DSB;
};

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_main_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ delta,
    float* __restrict__ dq_acc, uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int N, int n_kblk, int total,
    float c, float scale) {
  using S = BwdShape<D>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[S::LDSB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int g = lane >> 4, gi = lane & 15;
  const int dsub = g & 1, er = gi >> 2, qq = gi & 3;
  const int work = xcd_remap(blockIdx.x, total);
  const int bh = work / n_kblk, kblk = work - bh * n_kblk;
  const size_t head = (size_t)bh * N * D;
  const size_t hrow = (size_t)bh * N;
  const int k0 = kblk * BCK;
  const int krow = wave * 32 + l32;  // this lane's key within the block
  const int key = k0 + krow;
  const bool key_ok = key < N;
  const bool key_tail = k0 + BCK > N;

  // K and V fragments of this lane's key: B operands of S = Q K^T and dP = dO V^T.
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) {
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (key_ok) {
      a = *reinterpret_cast<const u32x4*>(K + head + (size_t)key * D + cc * 16 + h * 8);
      b = *reinterpret_cast<const u32x4*>(V + head + (size_t)key * D + cc * 16 + h * 8);
    }
    kf[cc] = as_bf16x8(a);
    vf[cc] = as_bf16x8(b);
  }
  // The whole K block in LDS: B operand (transposing reads) of dQ = dS K.
  unsigned char* Ks = smem + S::OFF_K;
#pragma unroll
  for (int r = 0; r < S::KCPT; ++r) {
    const int id = tid + r * kThreads;
    const int row = id / (D / 8), ch = id - row * (D / 8);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (k0 + row < N) v = *reinterpret_cast<const u32x4*>(K + head + (size_t)(k0 + row) * D + ch * 8);
    lds_write_b128(Ks, tile_off(row, ch * 8, S::ROWB), v);
  }

  f32x16 dvacc[D / 32], dkacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dvacc[db] = f32x16{};
    dkacc[db] = f32x16{};
  }

  const int nq = (N + BRQ - 1) / BRQ;
  u32x4 qst[S::QCPT], dost[S::QCPT];
  float lst = 0.f, dst = 0.f;

  auto gload = [&](int i) {
    const int q0 = i * BRQ;
#pragma unroll
    for (int r = 0; r < S::QCPT; ++r) {
      const int id = tid + r * kThreads;
      const int row = id / (D / 8), ch = id - row * (D / 8);
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (q0 + row < N) {
        a = *reinterpret_cast<const u32x4*>(Q + head + (size_t)(q0 + row) * D + ch * 8);
        b = *reinterpret_cast<const u32x4*>(dO + head + (size_t)(q0 + row) * D + ch * 8);
      }
      qst[r] = a;
      dost[r] = b;
    }
    if (tid < BRQ) {
      const int q = q0 + tid;
      lst = q < N ? LSE[hrow + q] * kLog2e : 0.f;
      dst = q < N ? delta[hrow + q] : 0.f;
    }
  };
  auto lstore = [&](int buf) {
    unsigned char* Qs = smem + S::OFF_Q + buf * S::QTILEB;
    unsigned char* dOs = smem + S::OFF_DO + buf * S::QTILEB;
#pragma unroll
    for (int r = 0; r < S::QCPT; ++r) {
      const int id = tid + r * kThreads;
      const int row = id / (D / 8), ch = id - row * (D / 8);
      const int off = tile_off(row, ch * 8, S::ROWB);
      lds_write_b128(Qs, off, qst[r]);
      lds_write_b128(dOs, off, dost[r]);
    }
    if (tid < BRQ) {
      reinterpret_cast<float*>(smem + S::OFF_L + buf * BRQ * 4)[tid] = lst;
      reinterpret_cast<float*>(smem + S::OFF_DL + buf * BRQ * 4)[tid] = dst;
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();

  unsigned char* dSt = smem + S::OFF_DS;

  for (int i = 0; i < nq; ++i) {
    const int buf = i & 1;
    if (i + 1 < nq) gload(i + 1);
    const unsigned char* Qs = smem + S::OFF_Q + buf * S::QTILEB;
    const unsigned char* dOs = smem + S::OFF_DO + buf * S::QTILEB;
    const float* L2 = reinterpret_cast<const float*>(smem + S::OFF_L + buf * BRQ * 4);
    const float* DL = reinterpret_cast<const float*>(smem + S::OFF_DL + buf * BRQ * 4);

    // ---- S = Q K^T and dP = dO V^T for 64 queries x this lane's key.
    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      sacc[mb] = f32x16{};
      pacc[mb] = f32x16{};
#pragma unroll
      for (int cc = 0; cc < D / 16; ++cc) {
        const int off = tile_off(mb * 32 + l32, cc * 16 + h * 8, S::ROWB);
        const bf16x8 aq = as_bf16x8(lds_read_b128(Qs, off));
        const bf16x8 ad = as_bf16x8(lds_read_b128(dOs, off));
        sacc[mb] = mfma32x32x16(aq, kf[cc], sacc[mb]);
        pacc[mb] = mfma32x32x16(ad, vf[cc], pacc[mb]);
      }
    }

    // ---- P = exp2(S * scale * log2 e - lse * log2 e), dS = P * (dP - delta).
    uint32_t ppk[2][8], dspk[2][8];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float4 l4 = *reinterpret_cast<const float4*>(L2 + mb * 32 + 8 * jj + 4 * h);
        const float4 d4 = *reinterpret_cast<const float4*>(DL + mb * 32 + 8 * jj + 4 * h);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
        float p[4], ds[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          p[ii] = __builtin_amdgcn_exp2f(fmaf(sacc[mb][4 * jj + ii], c, -lv[ii]));
          if (key_tail && !key_ok) p[ii] = 0.f;
          ds[ii] = p[ii] * (pacc[mb][4 * jj + ii] - dv[ii]);
        }
        ppk[mb][2 * jj] = pack_bf16(p[0], p[1]);
        ppk[mb][2 * jj + 1] = pack_bf16(p[2], p[3]);
        dspk[mb][2 * jj] = pack_bf16(ds[0], ds[1]);
        dspk[mb][2 * jj + 1] = pack_bf16(ds[2], ds[3]);
        // dS^T row of this key: queries mb*32 + 8jj + 4h .. +3.
        const u32x2 w = {dspk[mb][2 * jj], dspk[mb][2 * jj + 1]};
        *reinterpret_cast<u32x2*>(dSt + tile_off(krow, mb * 32 + 8 * jj + 4 * h, S::DSROWB)) = w;
      }

    // ---- dV^T += dO^T P and dK^T += Q^T dS (m = dim, n = key, k = query).
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const u32x4 bp = {ppk[mb][4 * c2], ppk[mb][4 * c2 + 1], ppk[mb][4 * c2 + 2], ppk[mb][4 * c2 + 3]};
        const u32x4 bs = {dspk[mb][4 * c2], dspk[mb][4 * c2 + 1], dspk[mb][4 * c2 + 2], dspk[mb][4 * c2 + 3]};
        const int row0 = mb * 32 + c2 * 16 + 4 * h + er;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int col = db * 32 + dsub * 16 + 4 * qq;
          const int o0 = tile_off(row0, col, S::ROWB), o1 = tile_off(row0 + 8, col, S::ROWB);
          const bf16x8 adot = as_bf16x8(lds_read_tr16_b64(dOs, o0), lds_read_tr16_b64(dOs, o1));
          const bf16x8 aqt = as_bf16x8(lds_read_tr16_b64(Qs, o0), lds_read_tr16_b64(Qs, o1));
          dvacc[db] = mfma32x32x16(adot, as_bf16x8(bp), dvacc[db]);
          dkacc[db] = mfma32x32x16(aqt, as_bf16x8(bs), dkacc[db]);
        }
      }

    __syncthreads();  // dS^T tile complete

    // ---- dQ share of this key block, dQ = dS K: (D/32) x 2 output tiles of
    // 32 queries x 32 dims split over the 4 waves; contraction over the 128
    // keys. A = dS (rows = queries) and B = K (columns = dims) both come from
    // transposing reads of key-major tiles. The accumulator holds 32
    // consecutive dims per row in a lane column, so each atomic instruction
    // updates two contiguous 128-byte row segments.
#pragma unroll
    for (int blk = wave; blk < (D / 32) * 2; blk += 4) {
      const int db = blk >> 1, nb = blk & 1;
      f32x16 qacc = f32x16{};
#pragma unroll
      for (int kc = 0; kc < BCK / 16; ++kc) {
        const int row0 = kc * 16 + 4 * h + er;
        const int sa = tile_off(row0, nb * 32 + dsub * 16 + 4 * qq, S::DSROWB);
        const int sb = tile_off(row0 + 8, nb * 32 + dsub * 16 + 4 * qq, S::DSROWB);
        const int ka = tile_off(row0, db * 32 + dsub * 16 + 4 * qq, S::ROWB);
        const int kb8 = tile_off(row0 + 8, db * 32 + dsub * 16 + 4 * qq, S::ROWB);
        const bf16x8 a = as_bf16x8(lds_read_tr16_b64(dSt, sa), lds_read_tr16_b64(dSt, sb));
        const bf16x8 b = as_bf16x8(lds_read_tr16_b64(Ks, ka), lds_read_tr16_b64(Ks, kb8));
        qacc = mfma32x32x16(a, b, qacc);
      }
      // Lane: dim db*32 + l32; rows: queries nb*32 + 8jj + 4h + ii.
      float* col = dq_acc + head + db * 32 + l32;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int q = i * BRQ + nb * 32 + 8 * jj + 4 * h + ii;
          if (q < N) unsafeAtomicAdd(col + (size_t)q * D, qacc[4 * jj + ii]);
        }
    }

    if (i + 1 < nq) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: dV = dV^T^T, dK = scale * dK^T^T (bf16, RNE). Lane: key, dims db*32 + 8jj + 4h + 0..3.
  if (key_ok) {
    uint16_t* dvrow = dV + head + (size_t)key * D;
    uint16_t* dkrow = dK + head + (size_t)key * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x16& a = dvacc[db];
        const f32x16& b = dkacc[db];
        const u32x2 wv = {pack_bf16(a[4 * jj], a[4 * jj + 1]), pack_bf16(a[4 * jj + 2], a[4 * jj + 3])};
        const u32x2 wk = {pack_bf16(b[4 * jj] * scale, b[4 * jj + 1] * scale),
                          pack_bf16(b[4 * jj + 2] * scale, b[4 * jj + 3] * scale)};
        *reinterpret_cast<u32x2*>(dvrow + db * 32 + 8 * jj + 4 * h) = wv;
        *reinterpret_cast<u32x2*>(dkrow + db * 32 + 8 * jj + 4 * h) = wk;
      }
  }
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int N, int d) {
  const size_t rows = (size_t)B * H * N;
  return align256(rows * 4) + align256(rows * (size_t)d * 4);
}

template <int D>
static hipError_t launch_bwd_stage_t(int stage, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     const uint16_t* o, const float* lse, const uint16_t* dO, uint16_t* dq,
                                     uint16_t* dk, uint16_t* dv, int B, int H, int N, float scale, void* workspace,
                                     hipStream_t stream) {
  const long rows = (long)B * H * N;
  float* delta = reinterpret_cast<float*>(workspace);
  float* dq_acc = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(workspace) + align256(rows * 4));
  if (stage == 0) {
    const long prep_threads = rows * 8;
    hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)((prep_threads + 255) / 256)), dim3(256), 0, stream, o,
                       dO, delta, dq_acc, rows);
  } else if (stage == 1) {
    const int n_kblk = (N + BCK - 1) / BCK;
    const int total = n_kblk * B * H;
    hipLaunchKernelGGL((bwd_main_kernel<D>), dim3(total), dim3(kThreads), 0, stream, q, k, v, dO, lse, delta, dq_acc,
                       dk, dv, N, n_kblk, total, scale * kLog2e, scale);
  } else {
    const long n8 = rows * D / 8;
    hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream, dq_acc, dq, n8,
                       scale);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_bf16_stage(int stage, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const uint16_t* o, const float* lse, const uint16_t* dO, uint16_t* dq, uint16_t* dk,
                                 uint16_t* dv, int B, int H, int N, int d, float scale, void* workspace,
                                 hipStream_t stream) {
  if (d == 64) return launch_bwd_stage_t<64>(stage, q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, workspace, stream);
  return launch_bwd_stage_t<128>(stage, q, k, v, o, lse, dO, dq, dk, dv, B, H, N, scale, workspace, stream);
}

}  // namespace attn
