// attn_fwd.hip - fused tiled attention forward for gfx950.
//
// Article "Selbstaufmerksamkeit, CUDA-Kernel und FlashAttention" (German
// edition of the self-attention / Triton / FlashAttention article,
// itimpress.au, 2026-11-15):
//   §1 "Scores"/"Attention" formulas  O = softmax(scale Q K^T) V, row-wise softmax;
//   §3 tiling bullet                  Q, K, V in on-chip tiles, only O written back;
//   §3 online-softmax bullet          running row max and normaliser rescale the
//                                     partial output as each K/V tile arrives;
//   §3 recompute bullet               the row statistic (here lse) is kept for the backward.
//
// 16-bit kernel (bf16 or fp16 storage and matrix-core operands, fp32
// accumulation and softmax): one workgroup = 4 or 8 waves; wave w owns 32*QB
// query rows.
// Everything is computed transposed, S^T = K Q^T and O^T = V^T P^T, so that a
// query is a lane column of every accumulator: row statistics (max, sum,
// rescale factor) are per-lane scalars, and the S^T accumulator converts to
// the B operand of the P*V product without leaving registers.
//   S^T  : A = K tile rows (LDS, 16-byte reads), B = Q fragment (registers)
//   O^T  : A = V^T (LDS, transposing 8-byte reads of the row-major V tile),
//          B = P^T (registers, 16-bit)
// K/V tiles go HBM -> LDS by direct DMA (no staging registers) into a ring
// of NS slots, so the next NS-1 tiles are in flight while one is computed.
//
// Three 16-bit kernels: fwd_kernel (every tile in one order: S, softmax,
// P V; masks, every head dim, short rows), fwd_sp_kernel (rows of whole
// 64-key tiles at d = 64 and 128, unmasked or causal: the
// same tiles and arithmetic per element, software-pipelined so that one
// wave's products overlap its own softmax) and fwd_pp_kernel (other unmasked
// rows of 1024 keys or more at d = 128: the two halves of the workgroup a
// phase apart, so that the matrix work of one wave of a SIMD overlaps the
// softmax of the other). Their outputs are equal bit for bit. fwd_f32_kernel
// is the fp32 forward on the vector ALU.
#include "attn_device.h"
#include "attn_kernels.h"

namespace attn {

namespace {

constexpr float kRescaleSlack = 8.0f;  // log2 units a row max may grow before O, l are rescaled

// Launch shape per head dim: 32-query blocks per wave (QB), 32-key blocks per
// K/V tile (KB) and K/V tiles in flight (NS, the LDS ring depth). Two waves
// share each SIMD (at most 256 registers per lane).
#ifndef FWD_WAVES_PER_EU
#define FWD_WAVES_PER_EU 2
#endif
// Long sequences use 8-wave workgroups (one per CU, two waves per SIMD, one
// K/V ring shared by all 8: each K/V tile crosses L2 -> LDS once per 8 waves);
// short ones 4-wave workgroups so that the row block does not overshoot N by
// much (see launch_fwd_e for where d = 32 and 64 switch).
#ifndef FWD_WAVES_LONG
#define FWD_WAVES_LONG 8
#endif
#ifndef FWD_LONG_N
#define FWD_LONG_N 1024
#endif
#ifndef FWD_LONG_N_SMALL_D
#define FWD_LONG_N_SMALL_D 8192
#endif
#ifndef FWD_QB64
#define FWD_QB64 2
#endif
#ifndef FWD_KB64
#define FWD_KB64 2
#endif
#ifndef FWD_NS64
#define FWD_NS64 2
#endif
// Rows shorter than FWD_LONG_N at d = 64 (the ViT heads): 4-wave workgroups
// of one 32-query block per wave (128 queries), a ring of 2 K/V tiles (32 KB
// of LDS) and three waves per SIMD (at most 168 registers, no spills), so
// that three workgroups share each CU: B=32, H=12, N=196 is 768 workgroups,
// one round of exactly three per CU. Measured (bit-identical outputs): 19.2
// -> 15.0 us per forward, causal B=16, H=12, N=197 15.6 -> 10.2 us. Two
// 32-query blocks per wave (one 256-query workgroup per head, 1.5 rounds of
// two per CU) were the previous shape; one block per wave with four waves
// per SIMD spills, and with a ring of 4 tiles only two workgroups fit per CU
// (24.7 and 19.3 us).
#ifndef FWD_QB64_SHORT
#define FWD_QB64_SHORT 1
#endif
#ifndef FWD_NS_SHORT
#define FWD_NS_SHORT 2
#endif
#ifndef FWD_WAVES_SHORT64
#define FWD_WAVES_SHORT64 4
#endif
#ifndef FWD_SHORT_WPE
#define FWD_SHORT_WPE 3
#endif
constexpr int fwd_waves_per_eu(int D, int QB, int WAVES) {
  return D == 64 && QB == 1 && WAVES == FWD_WAVES_SHORT64 ? FWD_SHORT_WPE : FWD_WAVES_PER_EU;
}
// Unmasked long rows use the ping-pong kernel at d = 128. At d = 64 (FWD_PP_D64)
// it measured 1.5 % faster than fwd_kernel but needs more than 256 registers
// per lane outside its main loop, and those spills double its HBM traffic,
// so d = 64 stays on fwd_kernel.
#ifndef FWD_PINGPONG
#define FWD_PINGPONG 1
#endif
// Software-pipelined forward for d = 64 rows without masks (N a multiple of 64, at least FWD_SP_MIN_N keys).
#ifndef FWD_SP
#define FWD_SP 1
#endif
#ifndef FWD_SP_MIN_N
#define FWD_SP_MIN_N 256
#endif
// The same pipelined forward at d = 128 (one query block per wave).
#ifndef FWD_SP128
#define FWD_SP128 1
#endif
// K and V tiles of the pipelined forward in separate LDS arrays, K first:
// at d_k = 128 no LDS read needs an address add (bit-identical; 14-16 vector
// instructions fewer per 32 products, B=2, H=16, N=16384 3594-3607 ->
// 3578-3586 us).
#ifndef FWD_SP_KV_SPLIT
#define FWD_SP_KV_SPLIT 1
#endif
// Causal rows at d_k = 128 on the pipelined forward (bit-identical to
// fwd_kernel): B=2, H=16, N=16384 2011 -> 1905 us, B=4, H=16, N=4096 282-303
// -> 272-275 us. At d_k = 64 (256-query workgroups against fwd_kernel's 128)
// it measured the same at N=4096 and 35 % slower at N=2048.
// Causal rows at d_k = 64 on the pipelined forward with one query block per
// wave (bit-identical to fwd_kernel): B=2, H=16, N=8192 316 -> 291 us, B=4,
// H=8, N=1024 17.4 -> 16.5 us, B=4, H=12, N=2048 43.7 -> 42.7 us, B=8, H=16,
// N=4096 315-318 -> 313 us; at N=256 3 % slower. Two blocks per wave (256-query
// workgroups) measured 35 % slower at N=2048 (more idle waves on the diagonal).
#ifndef FWD_MIX_BLOCKS
#define FWD_MIX_BLOCKS 1
#endif
#ifndef FWD_SP64_CAUSAL
#define FWD_SP64_CAUSAL 1
#endif
#ifndef FWD_SP64_CAUSAL_MIN_N
#define FWD_SP64_CAUSAL_MIN_N 1024
#endif
#ifndef FWD_SP_CAUSAL
#define FWD_SP_CAUSAL 1
#endif
#ifndef FWD_SP128_MIN_N
#define FWD_SP128_MIN_N 1024
#endif
// Schedule of the pipelined forward: operands read FWD_SP_AHEAD products ahead;
// FWD_SP_BARRIER keeps the compiler from moving work across chunks.
#ifndef FWD_SP_AHEAD
#define FWD_SP_AHEAD 2
#endif
#ifndef FWD_SP_BARRIER
#define FWD_SP_BARRIER 1
#endif
// FWD_SP_PIN keeps each chunk's exponentials in the chunk (see weight_pair).
// Measured, bit-identical outputs: B=2, H=16, N=16384, d_k=128 3710 -> 3580
// us, B=8, H=16, N=4096, d_k=64 546 -> 540 us (means of two runs each). Also
// pinning the row sums (FWD_SP_PIN 2) measured 2.5 % slower at d_k = 128, and
// reading operands 3 or 4 products ahead (FWD_SP_AHEAD) changed nothing.
// At d_k = 128 (two products per chunk) each chunk is split in two, one
// product and one exponential each, so that one wave's vector work fits in
// the shadow of its own products: bit-identical, B=2, H=16, N=16384
// 3447-3508 -> 3365-3434 us, B=4, H=16, N=4096 455-478 -> 446-448 us.
#ifndef FWD_SP_FINE
#define FWD_SP_FINE 1
#endif
#ifndef FWD_SP_PIN
#define FWD_SP_PIN 1
#endif
#ifndef FWD_PP_D64
#define FWD_PP_D64 0
#endif
#ifndef FWD_PP_QB64
#define FWD_PP_QB64 2
#endif
#ifndef FWD_PP_KB64
#define FWD_PP_KB64 2
#endif
#ifndef FWD_PP_QB128
#define FWD_PP_QB128 1
#endif
#ifndef FWD_PP_KB128
#define FWD_PP_KB128 2
#endif
#ifndef FWD_QB128
#define FWD_QB128 1
#endif
#ifndef FWD_KB128
#define FWD_KB128 2
#endif
#ifndef FWD_NS128
#define FWD_NS128 2
#endif

template <int D, int QB, int KB, int NS, int WAVES>
struct FwdShape {
  static constexpr int THREADS = WAVES * 64;
  static constexpr int BR = WAVES * 32 * QB;                  // query rows per workgroup
  static constexpr int BC = 32 * KB;                          // keys per K/V tile
  static constexpr int ROWB = D * 2;                          // bytes per K/V row
  static constexpr int TILEB = BC * ROWB;                     // bytes per K or V tile
  static constexpr int DMA_PER_WAVE = BC * D / 8 / THREADS;   // 16-byte DMA instructions per wave per tensor
  static constexpr int LDSB = NS * 2 * TILEB;                 // ring of NS (K, V) tile pairs
  static_assert(DMA_PER_WAVE >= 1 && (BC * D / 8) % THREADS == 0,
                "every lane takes part in each tile DMA, the same number of times");
};

template <class E, int D, int QB, int KB, int NS, int WAVES>
__global__ __launch_bounds__(WAVES * 64)
__attribute__((amdgpu_waves_per_eu(fwd_waves_per_eu(D, QB, WAVES), fwd_waves_per_eu(D, QB, WAVES))))
void fwd_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                     uint16_t* __restrict__ O, float* __restrict__ LSE, int N, int n_qblk, int total, float c,
                     uint32_t qsign, const int* __restrict__ kv_len, int H, int causal, Strides sq, Strides so) {
  using S = FwdShape<D, QB, KB, NS, WAVES>;
  static_assert(NS >= 2 && NS <= 4, "K/V ring of 2 to 4 tiles");
  // One LDS array per ring slot (K tile then V tile), addressed with a
  // compile-time slot index: the compiler can then tell a DMA into one slot
  // from the transposing reads of another, and does not make those reads wait
  // for the tile in flight (with one array it waits for every outstanding DMA).
  __shared__ __attribute__((aligned(16))) unsigned char ring0[2 * S::TILEB];
  __shared__ __attribute__((aligned(16))) unsigned char ring1[2 * S::TILEB];
  __shared__ __attribute__((aligned(16))) unsigned char ring2[NS > 2 ? 2 * S::TILEB : 16];
  __shared__ __attribute__((aligned(16))) unsigned char ring3[NS > 3 ? 2 * S::TILEB : 16];
  auto slot_base = [&](auto r_) __attribute__((always_inline)) -> unsigned char* {
    constexpr int R = decltype(r_)::value;
    if constexpr (R == 0) return ring0;
    else if constexpr (R == 1) return ring1;
    else if constexpr (R == 2) return ring2;
    else return ring3;
  };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int g = lane >> 4, gi = lane & 15;
  const int dsub = g & 1, er = gi >> 2, qq = gi & 3;
  const int work = xcd_remap(blockIdx.x, total);
  int bh, qblk;  // causal: the last row blocks have the most keys and are handed out first
  work_order(work, total, n_qblk, causal != 0, true, bh, qblk);
  // Heads of two row blocks, no causal mask: the block order alternates
  // between groups of 32 works, so that the workgroups resident on one CU
  // (works 32 apart on an XCD) hold first and second blocks of their heads in
  // turn rather than all first or all second ones (FWD_MIX_BLOCKS). Measured
  // (identical results): B=32, H=12, N=196 14.6-14.8 -> 14.0-14.6 us, B=64,
  // H=12, N=100 11.3-11.6 -> 11.2-11.5 us.
  if (FWD_MIX_BLOCKS && !causal && n_qblk == 2 && ((work / 32) & 1)) qblk ^= 1;
  const size_t hq = head_off(sq, bh, H);  // Q, K and V share one layout
  const uint16_t* Qh = Q + hq;
  const uint16_t* Kh = K + hq;
  const uint16_t* Vh = V + hq;
  const Rsrc rK = make_rsrc(Kh), rV = make_rsrc(Vh);
    const int qw0 = qblk * S::BR + wave * 32 * QB;

  // Visible keys of query q: j < klim(q) with klim(q) = min(kv, q + 1) under
  // the causal mask and kv otherwise (kv = valid keys of this batch entry).
  const int kv = kv_len ? min(max(kv_len[bh / H], 0), N) : N;
  const int cshift = causal ? 0 : N;  // klim(q) = min(kv, q + 1 + cshift); q + 1 + N > kv for every q
  auto klim = [&](int q) { return min(kv, q + 1 + cshift); };

  // Q fragments: B operand of S^T = K Q^T (lane: query l32, dims 16cc + 8h + 0..7).
  // A negative scale is folded into Q (exact sign flip) so that c >= 0.
  u32x4 qf[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int q = qw0 + qb * 32 + l32;
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (q < N) v = *reinterpret_cast<const u32x4*>(Qh + q * sq.n + cc * 16 + h * 8);  // q * n < 2^31 (host check)
      v ^= qsign;
      qf[qb][cc] = v;
    }
  }

  f32x16 oacc[QB][D / 32];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[qb][db] = f32x16{};
  }

  // Tiles this workgroup reads, tiles every query of the workgroup sees in
  // full (no mask), and the tiles this wave sees any key of.
  const int ntiles = (klim(qblk * S::BR + S::BR - 1) + S::BC - 1) / S::BC;
  const int nfull_wg = klim(qblk * S::BR) / S::BC;
  const int nvis_w = (klim(qw0 + 32 * QB - 1) + S::BC - 1) / S::BC;

  // K/V tile j -> ring slot R = j % NS by DMA. Wave w fills a contiguous run
  // of 16-byte LDS slots; the lane writing slot (row, s) fetches global chunk
  // s ^ swz(row), which yields the swizzled layout tile_off() addresses.
  // Rows past N re-read row N-1 (finite data; their scores are masked below).
  auto dma_tile = [&](int j, auto r_) __attribute__((always_inline)) {
    unsigned char* Ks = slot_base(r_);
    unsigned char* Vs = Ks + S::TILEB;
#pragma unroll
    for (int r = 0; r < S::DMA_PER_WAVE; ++r) {
      const int slot0 = (wave * S::DMA_PER_WAVE + r) * 64;
      const int p = slot0 + lane;
      const int row = p / (D / 8), chunk = (p - row * (D / 8)) ^ swz<S::ROWB>(row);
      const int key = min(j * S::BC + row, N - 1);
      const uint32_t off = (uint32_t)(key * sq.n + chunk * 8) * 2u;
      dma16(rK, off, Ks + slot0 * 16);
      dma16(rV, off, Vs + slot0 * 16);
    }
  };
  // Wait until tile j has landed, given that tiles up to min(j + NS - 2, ntiles - 1)
  // have been issued after it (each tile is 2 * DMA_PER_WAVE instructions per wave).
  auto wait_tile = [&](int j) {
    constexpr int PER = 2 * S::DMA_PER_WAVE;
    const int after = min(j + NS - 2, ntiles - 1) - j;
    if (NS >= 4 && after >= 2)
      wait_vmem_below<(NS >= 4 ? 2 * PER : 0)>();
    else if (NS >= 3 && after >= 1)
      wait_vmem_below<(NS >= 3 ? PER : 0)>();
    else
      wait_vmem_below<0>();
  };

  // Tile j with its ring slot as a compile-time constant.
  auto with_slot = [&](int j, auto&& f) __attribute__((always_inline)) {
    static_for<0, NS>([&](auto s_) __attribute__((always_inline)) {
      if (j % NS == decltype(s_)::value) f(s_);
    });
  };
  static_for<0, NS - 1>([&](auto s_) __attribute__((always_inline)) {
    if (decltype(s_)::value < ntiles) dma_tile(decltype(s_)::value, s_);
  });
  if (ntiles > 0) wait_tile(0);
  __syncthreads();

  // One K/V tile. MASKED tiles (the partial last tile, key padding, the
  // causal diagonal) drop each lane's invisible keys from the row max and give
  // them probability 0; fully visible tiles carry no masking code at all.
  // Per-lane byte offsets of the operand reads within a tile for key block 0:
  // K rows l32 (chunk 2cc + h) and the transposing V reads of rows 4h + er
  // (+ 8). The swizzle depends only on a row's low 4 bits, so key blocks,
  // 16-row halves and the ring slot (SLOT = j % NS, a compile-time constant)
  // are immediate offsets of the reads.
  int koff[D / 16], voff[2][D / 32];
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) koff[cc] = tile_off<S::ROWB>(l32, cc * 16 + h * 8);
#pragma unroll
  for (int hi = 0; hi < 2; ++hi)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) voff[hi][db] = tile_off<S::ROWB>(4 * h + er + 8 * hi, db * 32 + dsub * 16 + 4 * qq);
  auto tile = [&](int j, auto masked, auto slot_c) {
    constexpr bool MASKED = decltype(masked)::value;
    constexpr int SLOT = decltype(slot_c)::value;
    const unsigned char* Ks = slot_base(slot_c);
    const unsigned char* Vs = Ks + S::TILEB;
    int kvalid[QB];  // visible keys of this tile, per row block (MASKED only)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) kvalid[qb] = klim(qw0 + qb * 32 + l32) - j * S::BC;
    // 32-key blocks of this tile any query of the wave sees (wave-uniform: the
    // wave's last query sees the most keys). In a masked tile the blocks past
    // it are skipped whole: no products, no exponentials, no row-sum terms.
    // (Only masked tiles carry the test: a branch in the unmasked loop costs
    // more than it saves.)
    int kbv = KB;
    if (MASKED) kbv = min(KB, max(1, (klim(qw0 + 32 * QB - 1) - j * S::BC + 31) >> 5));

    // ---- S^T tile: BC keys x (32*QB) queries, fp32 accumulate.
    f32x16 sacc[QB][KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sacc[qb][kb] = f32x16{};
      if (MASKED && kb >= kbv) continue;
#pragma unroll
      for (int cc = 0; cc < D / 16; ++cc) {
        const u32x4 a = lds_read_b128(Ks, kb * 32 * S::ROWB + koff[cc]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sacc[qb][kb] = E::mfma(a, qf[qb][cc], sacc[qb][kb]);
      }
    }

    if (MASKED) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          if (kb >= kbv) continue;
          const int key = kb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            if (key >= kvalid[qb]) sacc[qb][kb][e] = -INFINITY;
        }
    }

    // ---- online softmax: running max in log2 units of the scaled score.
    // The reference point m_run only moves when the tile max exceeds it by
    // more than kRescaleSlack; any reference point gives the same softmax
    // (it cancels between O and l), so skipping small moves only bounds the
    // probabilities by 2^kRescaleSlack and saves the O rescale. The decision
    // is taken per 32-query block: when any lane of the wave needs a move,
    // every lane of that block moves its reference to its own maximum.
    float mnew[QB];
    bool need[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // NaN-propagating maximum (v_maximum3_f32): no canonicalisation of the
      // MFMA results is needed, unlike fmaxf. Masked tiles skip the key blocks
      // they did not compute (their accumulators hold zeros).
      float mx;
      if (!MASKED) {
        float xs[KB * 16];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) xs[kb * 16 + e] = sacc[qb][kb][e];
        mx = max_tree<KB * 16>(xs);
      } else {
        mx = sacc[qb][0][0];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          if (kb >= kbv) continue;
#pragma unroll
          for (int e = (kb == 0 ? 1 : 0); e < 16; e += 2)
            mx = (e + 1 < 16) ? fmax3(mx, sacc[qb][kb][e], sacc[qb][kb][e + 1]) : fmax2(mx, sacc[qb][kb][e]);
        }
      }
      mx = halves_max(mx) * c;
      mnew[qb] = fmaxf(m_run[qb], mx);
      need[qb] = mnew[qb] > m_run[qb] + kRescaleSlack;
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (__builtin_amdgcn_ballot_w64(need[qb])) {
        // A lane that has seen no visible key yet keeps max -inf (alpha = 1).
        const float alpha = mnew[qb] == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[qb] - mnew[qb]);
        m_run[qb] = mnew[qb];
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[qb][db] *= alpha;
      }
    }

    // ---- probabilities (16-bit) and their row sums. pb[qb][kb][c2] is directly
    // the B operand of the P V product for keys kb*32 + 16*c2 + (0..15).
    u32x4 pb[QB][KB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float nm = -m_run[qb];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          if (MASKED && kb >= kbv) continue;
          float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[qb][kb][e], c, nm));
          float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[qb][kb][e + 1], c, nm));
          if (MASKED) {
            const int key = kb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
            if (key >= kvalid[qb]) p0 = 0.f;
            if (key + 1 >= kvalid[qb]) p1 = 0.f;
          }
          const uint32_t w = E::pack(p0, p1);
          pb[qb][kb][e >> 3][(e >> 1) & 3] = w;
          l_run[qb] = E::sum_pair(w, l_run[qb]);
        }
    }

    // ---- O^T += V^T P^T.
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          if (MASKED && kb >= kbv) continue;
          const int rows = (kb * 32 + c2 * 16) * S::ROWB;
          const u32x2 lo = lds_read_tr16_b64(Vs, rows + voff[0][db]);
          const u32x2 hi = lds_read_tr16_b64(Vs, rows + voff[1][db]);
          const u32x4 a = cat(lo, hi);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = E::mfma(a, pb[qb][kb][c2], oacc[qb][db]);
        }
  };

  // Tiles every query of the workgroup sees in full run one single-path
  // loop. In the rest each wave runs the masked tile or, past its last
  // visible key, nothing; all waves still take part in every DMA and barrier.
  // The single-path loop is unrolled by NS (tile j in ring slot j % NS).
  auto full_tile = [&](int j, auto slot_c) __attribute__((always_inline)) {
    if (j + NS - 1 < ntiles) dma_tile(j + NS - 1, IntC<(decltype(slot_c)::value + NS - 1) % NS>{});
    tile(j, BoolC<false>{}, slot_c);
    if (j + 1 < ntiles) wait_tile(j + 1);
    __syncthreads();
  };
  int j = 0;
  for (; j + NS <= nfull_wg; j += NS)
    static_for<0, NS>([&](auto s_) __attribute__((always_inline)) { full_tile(j + decltype(s_)::value, s_); });
  for (; j < nfull_wg; ++j) with_slot(j, [&](auto s_) __attribute__((always_inline)) { full_tile(j, s_); });
  for (; j < ntiles; ++j) {
    if (j + NS - 1 < ntiles)
      with_slot(j + NS - 1, [&](auto s_) __attribute__((always_inline)) { dma_tile(j + NS - 1, s_); });
    if (j < nvis_w)  // masks are no-ops on the tiles this wave sees in full
      with_slot(j, [&](auto s_) __attribute__((always_inline)) { tile(j, BoolC<true>{}, s_); });
    if (j + 1 < ntiles) {
      wait_tile(j + 1);
      __syncthreads();
    }
  }

  // ---- epilogue: O = O^T / l (16-bit, RNE), lse = ln 2 * (m + log2 l). A row
  // with no visible key (l = 0) gets O = 0 and lse = -inf.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = halves_sum(l_run[qb]);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const int q = qw0 + qb * 32 + l32;
    if (q < N) {
      uint16_t* orow = O + head_off(so, bh, H) + q * so.n;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x16& a = oacc[qb][db];
          u32x2 w = {E::pack(a[4 * jj] * inv, a[4 * jj + 1] * inv), E::pack(a[4 * jj + 2] * inv, a[4 * jj + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * jj + 4 * h) = w;
        }
      if (h == 0) LSE[(size_t)bh * N + q] = lt > 0.f ? (m_run[qb] + log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

// ------------------------------------------------------------------------
// Ping-pong forward (long rows, no mask). The same tiles and the same
// arithmetic per element as fwd_kernel, in a different order: each wave's
// work on K/V tile j is split into a matrix-core phase (O^T += V_{j-1}^T
// P_{j-1}^T, then S_j^T = K_j Q^T) and a vector phase (the online softmax of
// S_j, giving P_j). Waves 0-3 and 4-7 run half a tile apart, separated by a
// workgroup barrier per phase, so that in every phase one wave of each SIMD
// feeds the matrix core while the other computes exponentials. The matrix
// phase runs at raised wave priority, so the arbiter issues the next matrix
// instruction as soon as it can and fills the gaps with the other wave's
// vector work.
//
// Phase schedule (slot s, barrier after every slot but the last): group g
// (= wave / 4) runs the matrix phase of tile j in slot 2j + g and the vector
// phase of tile j in slot 2j + 1 + g, for j = 0 .. ntiles (the last matrix
// phase only adds P V of the last tile). The K/V ring holds four tiles: each
// wave fetches its share of tile j + 2 during its matrix phase j, right after
// its transposing reads of V_{j-1}, and waits for it at the start of its
// matrix phase j + 1, so tile u is complete before the barrier that ends slot
// 2u - 1. K of tile u is read in slots 2u and 2u + 1, V in slots 2u + 2 and
// 2u + 3, and its ring slot is refilled (tile u + 4) from slot 2u + 4 on.
// Only raw s_barrier is used between phases: a fence would wait for the
// tiles in flight.
// ------------------------------------------------------------------------
constexpr int kPPWaves = 8;
constexpr int kPPRing = 4;

template <class E, int D, int QB, int KB>
__global__ __launch_bounds__(kPPWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_pp_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                   uint16_t* __restrict__ O, float* __restrict__ LSE, int N, int n_qblk, int total, float c,
                   uint32_t qsign, int H, Strides sq, Strides so) {
  using S = FwdShape<D, QB, KB, kPPRing, kPPWaves>;
  constexpr int NS = kPPRing;
  __shared__ __attribute__((aligned(16))) unsigned char smem[S::LDSB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = wave >> 2;
  const int h = lane >> 5, l32 = lane & 31;
  const int g = lane >> 4, gi = lane & 15;
  const int dsub = g & 1, er = gi >> 2, qq = gi & 3;
  const int work = xcd_remap(blockIdx.x, total);
  const int bh = work / n_qblk, qblk = work - bh * n_qblk;
  const size_t hq = head_off(sq, bh, H);
  const uint16_t* Qh = Q + hq;
  const uint16_t* Kh = K + hq;
  const uint16_t* Vh = V + hq;
  const Rsrc rK = make_rsrc(Kh), rV = make_rsrc(Vh);
  const int qw0 = qblk * S::BR + wave * 32 * QB;

  u32x4 qf[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int q = qw0 + qb * 32 + l32;
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (q < N) v = *reinterpret_cast<const u32x4*>(Qh + q * sq.n + cc * 16 + h * 8);
      v ^= qsign;
      qf[qb][cc] = v;
    }
  }

  f32x16 oacc[QB][D / 32];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[qb][db] = f32x16{};
  }

  const int ntiles = (N + S::BC - 1) / S::BC;
  const int tail = N - (ntiles - 1) * S::BC;  // valid keys of the last tile (1 .. BC)

  // Tile j into ring slot R (= j % NS).
  auto dma_tile = [&](int j, auto r_) __attribute__((always_inline)) {
    constexpr int R = decltype(r_)::value;
    unsigned char* Ks = smem + R * 2 * S::TILEB;
    unsigned char* Vs = Ks + S::TILEB;
#pragma unroll
    for (int r = 0; r < S::DMA_PER_WAVE; ++r) {
      const int slot0 = (wave * S::DMA_PER_WAVE + r) * 64;
      const int p = slot0 + lane;
      const int row = p / (D / 8), chunk = (p - row * (D / 8)) ^ swz<S::ROWB>(row);
      const int key = min(j * S::BC + row, N - 1);
      const uint32_t off = (uint32_t)(key * sq.n + chunk * 8) * 2u;
      dma16(rK, off, Ks + slot0 * 16);
      dma16(rV, off, Vs + slot0 * 16);
    }
  };
  // Phase boundary: this wave's LDS reads have returned, then all 8 waves meet.
  auto phase_end = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  f32x16 sacc[QB][KB];
  u32x4 pb[QB][KB][2];

  // Matrix-core phase of tile j in chunks of 8 products with D/16 operand
  // fragments each: chunks 0 .. KB-1 are O^T += V_{j-1}^T P_{j-1}^T for key
  // block kb (HAS_PV, j >= 1), chunks KB .. 2KB-1 are S_j^T for key block kb
  // (HAS_S, j < ntiles). The operands of chunk c + 1 are read from LDS while
  // chunk c runs; scheduling barriers keep the compiler from hoisting every
  // read of the phase to its top (which would need registers for all of them).
  constexpr int NOP = D / 16;
  // Per-lane byte offsets of the operand reads within a tile, for key block
  // 0: K rows l32 (chunk 2cc + h), and the transposing V reads of rows
  // 4h + er (+ 8). The swizzle depends only on a row's low 4 bits, so rows
  // 16m further on are these offsets plus 16m rows: key blocks, 16-row halves
  // and ring slots are immediate offsets of the LDS reads.
  int koff[NOP], voff[2][D / 32];
#pragma unroll
  for (int cc = 0; cc < NOP; ++cc) koff[cc] = tile_off<S::ROWB>(l32, cc * 16 + h * 8);
#pragma unroll
  for (int hi = 0; hi < 2; ++hi)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) voff[hi][db] = tile_off<S::ROWB>(4 * h + er + 8 * hi, db * 32 + dsub * 16 + 4 * qq);

  // Operands of chunk C of the matrix phase whose K tile sits in ring slot RK
  // (and V tile of the previous tile in slot (RK + NS - 1) % NS).
  auto load_chunk = [&](auto cc_, auto rk_, u32x4 (&a)[NOP]) __attribute__((always_inline)) {
    constexpr int C = decltype(cc_)::value, RK = decltype(rk_)::value;
    if constexpr (C < KB) {
      constexpr int VB = ((RK + NS - 1) % NS) * 2 * S::TILEB + S::TILEB;
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int rowb = VB + (C * 32 + c2 * 16) * S::ROWB;
          const u32x2 lo = lds_read_tr16_b64(smem, rowb + voff[0][db]);
          const u32x2 hi = lds_read_tr16_b64(smem, rowb + voff[1][db]);
          a[c2 * (D / 32) + db] = cat(lo, hi);
        }
    } else {
      constexpr int KBASE = RK * 2 * S::TILEB + (C - KB) * 32 * S::ROWB;
#pragma unroll
      for (int cc = 0; cc < NOP; ++cc) a[cc] = lds_read_b128(smem, KBASE + koff[cc]);
    }
  };
  auto run_chunk = [&](auto cc_, const u32x4 (&a)[NOP]) __attribute__((always_inline)) {
    constexpr int C = decltype(cc_)::value;
    if constexpr (C < KB) {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = E::mfma(a[c2 * (D / 32) + db], pb[qb][C][c2], oacc[qb][db]);
    } else {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sacc[qb][C - KB] = f32x16{};
#pragma unroll
      for (int cc = 0; cc < NOP; ++cc)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sacc[qb][C - KB] = E::mfma(a[cc], qf[qb][cc], sacc[qb][C - KB]);
    }
  };
  // `fetch` runs once every transposing read of V in the phase has been
  // issued (the compiler makes a transposing LDS read wait for all of the
  // wave's outstanding LDS DMA, so a fetch issued before them would be waited
  // for at once).
  auto mfma_phase = [&](auto has_pv, auto has_s, auto rk_, auto&& fetch) __attribute__((always_inline)) {
    constexpr int C0 = decltype(has_pv)::value ? 0 : KB;
    constexpr int C1 = decltype(has_s)::value ? 2 * KB : KB;
    u32x4 buf[2][NOP];
    if constexpr (C0 == KB) fetch();
    load_chunk(IntC<C0>{}, rk_, buf[0]);
    static_for<C0, C1>([&](auto cc_) __attribute__((always_inline)) {
      constexpr int C = decltype(cc_)::value;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (C + 1 == KB) fetch();
      if constexpr (C + 1 < C1) load_chunk(IntC<C + 1>{}, rk_, buf[(C + 1 - C0) & 1]);
      run_chunk(cc_, buf[(C - C0) & 1]);
    });
    __builtin_amdgcn_sched_barrier(0);
  };

  // Vector phase of tile j: online softmax of S_j (keys >= kvalid masked when MASKED).
  auto valu_phase = [&](auto masked, int kvalid) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    if (MASKED) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            if (key >= kvalid) sacc[qb][kb][e] = -INFINITY;
        }
    }
    float mnew[QB];
    bool need[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // (A running chain here: the three-operand tree of fwd_kernel measured
      // 2 % slower in this kernel at d = 128.)
      float mx = sacc[qb][0][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = (kb == 0 ? 1 : 0); e < 16; e += 2)
          mx = (e + 1 < 16) ? fmax3(mx, sacc[qb][kb][e], sacc[qb][kb][e + 1]) : fmax2(mx, sacc[qb][kb][e]);
      mx = halves_max(mx) * c;
      mnew[qb] = fmaxf(m_run[qb], mx);
      need[qb] = mnew[qb] > m_run[qb] + kRescaleSlack;
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (__builtin_amdgcn_ballot_w64(need[qb])) {
        const float alpha = mnew[qb] == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[qb] - mnew[qb]);
        m_run[qb] = mnew[qb];
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[qb][db] *= alpha;
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float nm = -m_run[qb];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[qb][kb][e], c, nm));
          float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[qb][kb][e + 1], c, nm));
          if (MASKED) {
            const int key = kb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
            if (key >= kvalid) p0 = 0.f;
            if (key + 1 >= kvalid) p1 = 0.f;
          }
          const uint32_t w = E::pack(p0, p1);
          pb[qb][kb][e >> 3][(e >> 1) & 3] = w;
          l_run[qb] = E::sum_pair(w, l_run[qb]);
        }
    }
  };

  // Matrix phase of tile j (ring slot R = j % NS) at raised priority. It
  // first waits for this wave's share of tile j + 1 (fetched in its previous
  // matrix phase) and fetches its share of tile j + 2 once its reads of V_{j-1}
  // are issued.
  auto matrix_slot = [&](auto has_pv, auto has_s, auto r_, int j) __attribute__((always_inline)) {
    constexpr int R = decltype(r_)::value;
    wait_vmem_below<0>();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    mfma_phase(has_pv, has_s, r_, [&]() __attribute__((always_inline)) {
      if (j + 2 < ntiles) dma_tile(j + 2, IntC<(R + 2) % NS>{});
    });
    __builtin_amdgcn_s_setprio(0);
  };
  auto vector_slot = [&](int j, auto may_mask) __attribute__((always_inline)) {
    if (decltype(may_mask)::value && j == ntiles - 1 && tail < S::BC)
      valu_phase(BoolC<true>{}, tail);
    else
      valu_phase(BoolC<false>{}, S::BC);
    phase_end();
  };
  // One whole tile j >= 1 in ring slot R.
  auto full_tile = [&](auto r_, int j, auto may_mask) __attribute__((always_inline)) {
    matrix_slot(BoolC<true>{}, BoolC<true>{}, r_, j);
    phase_end();
    vector_slot(j, may_mask);
  };

  // Prologue: tiles 0 and 1 resident before slot 0; group 1 sits out slot 0.
  dma_tile(0, IntC<0>{});
  if (ntiles > 1) dma_tile(1, IntC<1>{});
  wait_vmem_below<0>();
  __syncthreads();
  if (grp == 1) phase_end();
  matrix_slot(BoolC<false>{}, BoolC<true>{}, IntC<0>{}, 0);
  phase_end();
  vector_slot(0, BoolC<true>{});
  // Tiles 1 .. ntiles - 1, four per iteration (ring slots 1, 2, 3, 0) while
  // none of them is the last; then the remaining one to four.
  int j = 1;
  for (; j + 4 < ntiles; j += 4) {
    full_tile(IntC<1>{}, j, BoolC<false>{});
    full_tile(IntC<2>{}, j + 1, BoolC<false>{});
    full_tile(IntC<3>{}, j + 2, BoolC<false>{});
    full_tile(IntC<0>{}, j + 3, BoolC<false>{});
  }
  if (j < ntiles) full_tile(IntC<1>{}, j, BoolC<true>{});
  if (j + 1 < ntiles) full_tile(IntC<2>{}, j + 1, BoolC<true>{});
  if (j + 2 < ntiles) full_tile(IntC<3>{}, j + 2, BoolC<true>{});
  if (j + 3 < ntiles) full_tile(IntC<0>{}, j + 3, BoolC<true>{});
  // Last matrix phase: P V of tile ntiles - 1 (its V in ring slot (ntiles - 1) % NS).
  switch ((ntiles - 1) % NS) {
    case 0: matrix_slot(BoolC<true>{}, BoolC<false>{}, IntC<1>{}, ntiles); break;
    case 1: matrix_slot(BoolC<true>{}, BoolC<false>{}, IntC<2>{}, ntiles); break;
    case 2: matrix_slot(BoolC<true>{}, BoolC<false>{}, IntC<3>{}, ntiles); break;
    default: matrix_slot(BoolC<true>{}, BoolC<false>{}, IntC<0>{}, ntiles); break;
  }
  if (grp == 0) phase_end();

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = halves_sum(l_run[qb]);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const int q = qw0 + qb * 32 + l32;
    if (q < N) {
      uint16_t* orow = O + head_off(so, bh, H) + q * so.n;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x16& a = oacc[qb][db];
          u32x2 w = {E::pack(a[4 * jj] * inv, a[4 * jj + 1] * inv), E::pack(a[4 * jj + 2] * inv, a[4 * jj + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * jj + 4 * h) = w;
        }
      if (h == 0) LSE[(size_t)bh * N + q] = lt > 0.f ? (m_run[qb] + log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

// ------------------------------------------------------------------------
// Software-pipelined forward (rows without masks, N a multiple of 64; d = 64
// with two 32-query blocks per wave, d = 128 with one). The same tiles and
// the same arithmetic per element as fwd_kernel, issued so that every wave
// keeps the matrix cores and the vector ALU busy at once.
//
// A unit is one 32-query block of the wave against one 64-key tile: with two
// blocks tile j holds units (j, 0) and (j, 1), with one block tile j is unit
// j. While the vector ALU computes the softmax of unit u, the matrix cores
// compute S of unit u + 1 and O^T += V^T P^T of unit u - 1 (independent
// instructions in one stream, interleaved by the hardware). So S of tile
// j + 1 is read from LDS while V of tile j - 1 is still in use: the K/V ring
// holds four tiles, one LDS array per slot.
//
// The softmax is speculative: the weights are computed against the current
// reference maximum without first taking the tile's maximum. The reference
// only has to move when a weight exceeds 2^kRescaleSlack, and then the
// tile's share of the row sum exceeds it too; only then (ballot over the
// wave) the tile takes the full path of fwd_kernel: maximum, move, rescale
// and exponentials again. A tile that passes computed exactly the
// exponentials fwd_kernel computes, so the outputs are equal bit for bit.
// After a unit whose reference moved, the next unit of that query block
// takes the maximum first, as fwd_kernel does (the same result, without the
// wasted exponentials when the maximum keeps rising).
// ------------------------------------------------------------------------
constexpr int kSPRing = 4;
// Row-sum share of one tile above which the full path runs: below 2^kRescaleSlack
// by more than the rounding of the fp32 sum, so that no weight above that bound
// can pass unchecked.
constexpr float kSpecLimit = 128.0f;

// CAUSAL: the causal mask. The tiles every query of the workgroup sees in
// full (keys before its first query) run the pipelined units; the diagonal
// tiles after them run fwd_kernel's masked tile, one tile at a time.
template <class E, int D, int QB, int WAVES, bool CAUSAL>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_sp_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                   uint16_t* __restrict__ O, float* __restrict__ LSE, int N, int n_qblk, int total, float c,
                   uint32_t qsign, int H, Strides sq, Strides so) {
  static_assert((D == 64 && (QB == 1 || QB == 2)) || (D == 128 && QB == 1), "shapes with a register plan");
  constexpr int KB = 2, NS = kSPRing;
  using S = FwdShape<D, QB, KB, NS, WAVES>;
  constexpr int NDB = D / 32, NCC = D / 16;
  constexpr int NPV = KB * 2 * NDB;  // P V products per unit (key block, 16-key half, 32-dim block)
  constexpr int NSP = KB * NCC;      // S^T products per unit (key block, 16-dim chunk)
  constexpr int PPC = (NPV + NSP) / 16;  // products per chunk of a unit: 1 at d = 64, 2 at d = 128
  constexpr int PER = 2 * S::DMA_PER_WAVE;  // DMA instructions per wave per tile
#if FWD_SP_KV_SPLIT
  // K tiles of the four slots first, then the V tiles (declaration order is
  // allocation order): at d = 128 the K tiles fill the first 64 KB and every
  // K read reaches its slot through the 16-bit offset field; the V reads
  // reach theirs from per-lane offsets biased by 64 KB (below). One array per
  // tile keeps the copies into different tiles apart for the compiler's
  // wait placement.
  __shared__ __attribute__((aligned(16))) unsigned char kring0[S::TILEB];
  __shared__ __attribute__((aligned(16))) unsigned char kring1[S::TILEB];
  __shared__ __attribute__((aligned(16))) unsigned char kring2[S::TILEB];
  __shared__ __attribute__((aligned(16))) unsigned char kring3[S::TILEB];
  __shared__ __attribute__((aligned(16))) unsigned char vring0[S::TILEB];
  __shared__ __attribute__((aligned(16))) unsigned char vring1[S::TILEB];
  __shared__ __attribute__((aligned(16))) unsigned char vring2[S::TILEB];
  __shared__ __attribute__((aligned(16))) unsigned char vring3[S::TILEB];
  auto k_base = [&](auto r_) __attribute__((always_inline)) -> unsigned char* {
    constexpr int R = decltype(r_)::value % NS;
    if constexpr (R == 0) return kring0;
    else if constexpr (R == 1) return kring1;
    else if constexpr (R == 2) return kring2;
    else return kring3;
  };
  auto v_base = [&](auto r_) __attribute__((always_inline)) -> unsigned char* {
    constexpr int R = decltype(r_)::value % NS;
    if constexpr (R == 0) return vring0;
    else if constexpr (R == 1) return vring1;
    else if constexpr (R == 2) return vring2;
    else return vring3;
  };
  // Bias of the V offsets: the V tiles start after the four K tiles; past
  // 64 KB the offset field cannot hold the slot, so the per-lane offsets
  // carry the first 64 KB.
  constexpr int VBIAS = NS * S::TILEB >= 65536 ? 65536 : 0;
#else
  __shared__ __attribute__((aligned(16))) unsigned char ring0[2 * S::TILEB];
  __shared__ __attribute__((aligned(16))) unsigned char ring1[2 * S::TILEB];
  __shared__ __attribute__((aligned(16))) unsigned char ring2[2 * S::TILEB];
  __shared__ __attribute__((aligned(16))) unsigned char ring3[2 * S::TILEB];
  auto slot_base = [&](auto r_) __attribute__((always_inline)) -> unsigned char* {
    constexpr int R = decltype(r_)::value % NS;
    if constexpr (R == 0) return ring0;
    else if constexpr (R == 1) return ring1;
    else if constexpr (R == 2) return ring2;
    else return ring3;
  };
  auto k_base = [&](auto r_) __attribute__((always_inline)) -> unsigned char* { return slot_base(r_); };
  auto v_base = [&](auto r_) __attribute__((always_inline)) -> unsigned char* { return slot_base(r_) + S::TILEB; };
  constexpr int VBIAS = 0;
#endif

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int g = lane >> 4, gi = lane & 15;
  const int dsub = g & 1, er = gi >> 2, qq = gi & 3;
  const int work = xcd_remap(blockIdx.x, total);
  int bh, qblk;  // causal: the last row blocks have the most keys and are handed out first
  work_order(work, total, n_qblk, CAUSAL, true, bh, qblk);
  const size_t hq = head_off(sq, bh, H);
  const uint16_t* Qh = Q + hq;
  const uint16_t* Kh = K + hq;
  const uint16_t* Vh = V + hq;
  const Rsrc rK = make_rsrc(Kh), rV = make_rsrc(Vh);
  const int qw0 = qblk * S::BR + wave * 32 * QB;

  u32x4 qf[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int q = qw0 + qb * 32 + l32;
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (q < N) v = *reinterpret_cast<const u32x4*>(Qh + q * sq.n + cc * 16 + h * 8);
      v ^= qsign;
      qf[qb][cc] = v;
    }
  }

  f32x16 oacc[QB][D / 32];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[qb][db] = f32x16{};
  }

  // Pipelined tiles (N is a multiple of the tile; without the mask the
  // launcher checks nt >= 4) and tiles read: under the causal mask the
  // workgroup's first query sees the first nt in full (a multiple of
  // BR / 64: none, or at least 2), and its rows reach tile nt_dma - 1.
  const int nt = CAUSAL ? qblk * S::BR / S::BC : N / S::BC;
  const int nt_dma = CAUSAL ? min(N, (qblk + 1) * S::BR) / S::BC : nt;

  auto dma_tile = [&](int j, auto r_) __attribute__((always_inline)) {
    unsigned char* Ks = k_base(r_);
    unsigned char* Vs = v_base(r_);
#pragma unroll
    for (int r = 0; r < S::DMA_PER_WAVE; ++r) {
      const int slot0 = (wave * S::DMA_PER_WAVE + r) * 64;
      const int p = slot0 + lane;
      const int row = p / (D / 8), chunk = (p - row * (D / 8)) ^ swz<S::ROWB>(row);
      const int key = j * S::BC + row;
      const uint32_t off = (uint32_t)(key * sq.n + chunk * 8) * 2u;
      dma16(rK, off, Ks + slot0 * 16);
      dma16(rV, off, Vs + slot0 * 16);
    }
  };

  int koff[D / 16], voff[2][D / 32];
#pragma unroll
  for (int cc = 0; cc < D / 16; ++cc) koff[cc] = tile_off<S::ROWB>(l32, cc * 16 + h * 8);
#pragma unroll
  for (int hi = 0; hi < 2; ++hi)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      voff[hi][db] = tile_off<S::ROWB>(4 * h + er + 8 * hi, db * 32 + dsub * 16 + 4 * qq) + VBIAS;
      // Hidden from the optimiser, so that it cannot take the bias back out
      // of the register and into a per-read address add.
      if constexpr (VBIAS != 0) __asm__("" : "+v"(voff[hi][db]));
    }

  // One unit's work is issued as 16 chunks at d = 64, each one matrix
  // product, the exponentials of one pair of S^T entries and the LDS read of
  // the operand two products ahead, with scheduling barriers between chunks:
  // the compiler keeps them in order (left alone, it hoists every operand
  // read of the iteration and spills). At d = 128 a unit has twice the
  // products and the same exponentials: 32 chunks of one product and one
  // exponential each (16 chunks of two products with FWD_SP_FINE 0).
  // Products at d = 64: first P V of the previous unit (PV, 8:
  // key block, 16-key half, 32-dim block; the two 32-dim accumulators
  // alternate), then S^T of the next one (S, 8: the two key blocks' chains
  // alternate, 16-dim chunks in order). The kinds are not interleaved: the
  // compiler assumes transposing and plain LDS reads may complete out of
  // order, and waits for every read in flight when the two are mixed.
  // Operand of product m of a unit: V^T fragment (PV) or K fragment (S).
  auto pv_operand = [&](auto r_, int p) __attribute__((always_inline)) -> u32x4 {
    const unsigned char* Vs = v_base(r_);
    const int kb = p / (2 * NDB), c2 = (p / NDB) & 1, db = p % NDB;
    const int rows = (kb * 32 + c2 * 16) * S::ROWB - VBIAS;
    return cat(lds_read_tr16_b64(Vs, rows + voff[0][db]), lds_read_tr16_b64(Vs, rows + voff[1][db]));
  };
  auto s_operand = [&](auto r_, int sidx) __attribute__((always_inline)) -> u32x4 {
    const unsigned char* Ks = k_base(r_);
    return lds_read_b128(Ks, (sidx / NCC) * 32 * S::ROWB + koff[sidx % NCC]);
  };
  // Weights of entries 2i, 2i + 1 of query block QB_'s S^T tile (i = 0 .. 15).
  auto weight_pair = [&](auto qb_, int i, const f32x16 (&sv)[KB], u32x4 (&p)[KB][2], float& l)
                         __attribute__((always_inline)) {
    constexpr int QB_ = decltype(qb_)::value;
    const int kb = i >> 3, e = 2 * (i & 7);
    const float nm = -m_run[QB_];
    const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[kb][e], c, nm));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[kb][e + 1], c, nm));
    const uint32_t w = E::pack(p0, p1);
#if FWD_SP_PIN
    // An empty use of the pair here keeps its exponentials in this chunk: the
    // weights are first read after the unit, past the conditional O rescale,
    // and the compiler otherwise sinks all of them below the unit's products.
    __asm__ volatile("" : : "v"(w));
#endif
    p[kb][e >> 3][(e >> 1) & 3] = w;
    l = E::sum_pair(w, l);
#if FWD_SP_PIN > 1
    __asm__ volatile("" : : "v"(l));  // the same for the row sum
#endif
  };
  // The same pair in two steps, one exponential each, for chunks of one
  // product (FWD_SP_FINE).
  auto weight_first = [&](auto qb_, int i, const f32x16 (&sv)[KB]) __attribute__((always_inline)) -> float {
    constexpr int QB_ = decltype(qb_)::value;
    const int kb = i >> 3, e = 2 * (i & 7);
    const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[kb][e], c, -m_run[QB_]));
    __asm__ volatile("" : : "v"(p0));
    return p0;
  };
  auto weight_second = [&](auto qb_, int i, const f32x16 (&sv)[KB], float p0, u32x4 (&p)[KB][2], float& l)
                           __attribute__((always_inline)) {
    constexpr int QB_ = decltype(qb_)::value;
    const int kb = i >> 3, e = 2 * (i & 7);
    const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[kb][e + 1], c, -m_run[QB_]));
    const uint32_t w = E::pack(p0, p1);
    __asm__ volatile("" : : "v"(w));
    p[kb][e >> 3][(e >> 1) & 3] = w;
    l = E::sum_pair(w, l);
  };
  // The first step of fwd_kernel's softmax for one unit: the maximum of its
  // scores and, when the reference has to move (ballot over the wave), the
  // move. Returns the rescale factor for O and l (1 without a move) and
  // whether the reference moved (wave-uniform); the caller rescales O once
  // every product into it that predates the move has been issued.
  auto move_reference = [&](auto qb_, const f32x16 (&sv)[KB], float& alpha) __attribute__((always_inline)) -> bool {
    constexpr int QB_ = decltype(qb_)::value;
    float xs[KB * 16];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) xs[kb * 16 + e] = sv[kb][e];
    const float mx = halves_max(max_tree<KB * 16>(xs)) * c;
    const float mnew = fmaxf(m_run[QB_], mx);
    alpha = 1.f;
    if (__builtin_amdgcn_ballot_w64(mnew > m_run[QB_] + kRescaleSlack)) {
      alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[QB_] - mnew);
      m_run[QB_] = mnew;
      return true;
    }
    return false;
  };
  // The full path of fwd_kernel for one unit whose speculative weights failed
  // the check: maximum, reference move and rescale, weights again. Returns
  // whether the reference moved.
  auto softmax_slow = [&](auto qb_, const f32x16 (&sv)[KB], u32x4 (&p)[KB][2], float l_old, float& l)
                          __attribute__((always_inline)) -> bool {
    constexpr int QB_ = decltype(qb_)::value;
    float alpha;
    if (!move_reference(qb_, sv, alpha)) return false;
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[QB_][db] *= alpha;
    l = l_old * alpha;
#pragma unroll
    for (int i = 0; i < 16; ++i) weight_pair(qb_, i, sv, p, l);
    return true;
  };
  // Per query block: the last unit moved the reference. Then the next unit
  // takes the maximum first (fwd_kernel's order) instead of speculating: with
  // peaked scores the row maximum keeps rising for many tiles and most
  // speculative weights would be computed twice. Every row block starts with
  // a move (from -infinity).
  bool moved_last[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) moved_last[qb] = true;

  // One unit: softmax of query block QS (S^T in sv -> P^T in pw), with S^T of
  // query block QN against the K tile in slot RS into sn (HAS_S) and P V of
  // query block QP (P^T in pr) against the V tile in slot RV (HAS_PV).
  auto unit = [&](auto has_s, auto rs_, auto qn_, f32x16 (&sn)[KB], auto has_pv, auto rv_, auto qp_,
                  const u32x4 (&pr)[KB][2], auto qs_, const f32x16 (&sv)[KB], u32x4 (&pw)[KB][2])
                  __attribute__((always_inline)) {
    constexpr bool HS = decltype(has_s)::value, HP = decltype(has_pv)::value;
    constexpr int QN = decltype(qn_)::value, QP = decltype(qp_)::value, QS = decltype(qs_)::value;
    constexpr int NM = (HS ? NSP : 0) + (HP ? NPV : 0);
    // Product m: PV index m (m < NPV, HAS_PV), then S index m - NPV (or m
    // without PV products), S index t meaning key block t % KB and 16-dim
    // chunk t / KB (the key blocks' accumulation chains alternate).
    auto is_pv = [&](int m) { return HP && m < NPV; };
    auto s_index = [&](int m) { return HP ? m - NPV : m; };
    auto operand = [&](int m) __attribute__((always_inline)) -> u32x4 {
      if (is_pv(m)) return pv_operand(rv_, m);
      const int t = s_index(m);
      return s_operand(rs_, (t % KB) * NCC + t / KB);
    };
    if constexpr (HS) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sn[kb] = f32x16{};
    }
    const bool max_first = moved_last[QS];
    bool moved = false;
    float l_old = l_run[QS], alpha_first = 1.f;
    if (max_first) {
      moved = move_reference(qs_, sv, alpha_first);
      l_old *= alpha_first;
    }
    float l = l_old;
    constexpr int AH = FWD_SP_AHEAD, NO = AH + 1;  // operands read AH products ahead
    u32x4 ops[NO];
    static_for<0, AH>([&](auto a_) __attribute__((always_inline)) {
      if constexpr (decltype(a_)::value < NM) ops[decltype(a_)::value] = operand(decltype(a_)::value);
    });
    constexpr bool FINE = FWD_SP_FINE && PPC == 2;
    float p_first = 0.f;
    static_for<0, FINE ? 32 : 16>([&](auto i_) __attribute__((always_inline)) {
      constexpr int I = FINE ? decltype(i_)::value / 2 : decltype(i_)::value;
      constexpr int HALF = FINE ? decltype(i_)::value % 2 : 0;
      if (FWD_SP_BARRIER) __builtin_amdgcn_sched_barrier(0);
      static_for<0, FINE ? 1 : PPC>([&](auto u_) __attribute__((always_inline)) {
        constexpr int M = FINE ? decltype(i_)::value : I * PPC + decltype(u_)::value;
        if constexpr (M < NM) {
          constexpr bool PVM = HP && M < NPV;
          if constexpr (PVM) {
            constexpr int kb = M / (2 * NDB), c2 = (M / NDB) & 1, db = M % NDB;
            oacc[QP][db] = E::mfma(ops[M % NO], pr[kb][c2], oacc[QP][db]);
          } else {
            constexpr int T = HP ? M - NPV : M, kb = T % KB, cc = T / KB;
            sn[kb] = E::mfma(ops[M % NO], qf[QN][cc], sn[kb]);
          }
        }
        if constexpr (M + AH < NM) ops[(M + AH) % NO] = operand(M + AH);
      });
      if constexpr (!FINE)
        weight_pair(qs_, I, sv, pw, l);
      else if constexpr (HALF == 0)
        p_first = weight_first(qs_, I, sv);
      else
        weight_second(qs_, I, sv, p_first, pw, l);
    });
    __builtin_amdgcn_sched_barrier(0);
    // A maximum-first move rescales O now: with one query block per wave the
    // P V products of this unit went into the same accumulator, relative to
    // the old reference.
    if (max_first && moved) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[QS][db] *= alpha_first;
    }
    // After the maximum-first path the weights are those of fwd_kernel (at
    // most 2^kRescaleSlack each) and need no check.
    if (!max_first && __builtin_amdgcn_ballot_w64(!(l - l_old <= kSpecLimit)))
      moved = softmax_slow(qs_, sv, pw, l_old, l);
    moved_last[QS] = moved;
    l_run[QS] = l;
  };

  // Two query blocks per wave: at the end of tile j's first unit, tile j + 1
  // landed and visible to every wave, every wave done with tile j - 1 (its
  // slot takes tile j + 3). One block per wave: at the end of tile j's unit,
  // tile j + 2 landed and visible (the next unit computes its S^T), every
  // wave done with tile j - 1 (its V fed this unit's P V).
  auto boundary = [&](int j, auto r_) __attribute__((always_inline)) {
    constexpr int R = decltype(r_)::value;
    if constexpr (QB == 2) {
      if (j + 2 >= 3 && j + 2 < nt_dma)
        wait_vmem_below<PER>();
      else
        wait_vmem_below<0>();
    } else {
      wait_vmem_below<0>();
    }
    __syncthreads();
    if (j + 3 < nt_dma) dma_tile(j + 3, IntC<(R + 3) % NS>{});
  };

  // Two query blocks: S^T of blocks 0 and 1 (one tile apart) in sa / sb, P^T
  // of blocks 1 and 0 in pa / pb. One block: S^T and P^T of even tiles in sa
  // / pa, of odd tiles in sb / pb.
  f32x16 sa[KB], sb[KB];
  u32x4 pa[KB][2], pb[KB][2];
  // Tile j in ring slot R. FIRST: no P V of tile j - 1; LAST: no S of tile j + 1.
  auto tile = [&](int j, auto r_, auto first_, auto last_) __attribute__((always_inline)) {
    constexpr int R = decltype(r_)::value;
    constexpr bool FIRST = decltype(first_)::value, LAST = decltype(last_)::value;
    if constexpr (QB == 2) {
      // unit (j, 0): S^T(j, 1) -> sb, P V(j - 1, 1) from pa, softmax(j, 0): sa -> pb
      unit(BoolC<true>{}, r_, IntC<1>{}, sb, BoolC<!FIRST>{}, IntC<(R + NS - 1) % NS>{}, IntC<1>{}, pa, IntC<0>{}, sa,
           pb);
      boundary(j, r_);
      // unit (j, 1): S^T(j + 1, 0) -> sa, P V(j, 0) from pb, softmax(j, 1): sb -> pa
      unit(BoolC<!LAST>{}, IntC<(R + 1) % NS>{}, IntC<0>{}, sa, BoolC<true>{}, r_, IntC<0>{}, pb, IntC<1>{}, sb, pa);
    } else if constexpr (R % 2 == 0) {  // even tile (the ring has an even number of slots)
      // unit j: S^T(j + 1) -> sb, P V(j - 1) from pb, softmax(j): sa -> pa
      unit(BoolC<!LAST>{}, IntC<(R + 1) % NS>{}, IntC<0>{}, sb, BoolC<!FIRST>{}, IntC<(R + NS - 1) % NS>{}, IntC<0>{},
           pb, IntC<0>{}, sa, pa);
      boundary(j, r_);
    } else {
      // unit j: S^T(j + 1) -> sa, P V(j - 1) from pa, softmax(j): sb -> pb
      unit(BoolC<!LAST>{}, IntC<(R + 1) % NS>{}, IntC<0>{}, sa, BoolC<!FIRST>{}, IntC<(R + NS - 1) % NS>{}, IntC<0>{},
           pa, IntC<0>{}, sb, pb);
      boundary(j, r_);
    }
  };
  // S^T of unit (0, 0) and P V of the last unit, outside any tile.
  auto s_only = [&](auto r_, auto qb_, f32x16 (&acc)[KB]) __attribute__((always_inline)) {
    constexpr int QB_ = decltype(qb_)::value;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      acc[kb] = f32x16{};
#pragma unroll
      for (int cc = 0; cc < NCC; ++cc) acc[kb] = E::mfma(s_operand(r_, kb * NCC + cc), qf[QB_][cc], acc[kb]);
    }
  };
  auto pv_only = [&](auto r_, auto qb_, const u32x4 (&p)[KB][2]) __attribute__((always_inline)) {
    constexpr int QB_ = decltype(qb_)::value;
#pragma unroll
    for (int m = 0; m < NPV; ++m)
      oacc[QB_][m % NDB] = E::mfma(pv_operand(r_, m), p[m / (2 * NDB)][(m / NDB) & 1], oacc[QB_][m % NDB]);
  };

  // A diagonal tile under the causal mask, as fwd_kernel's masked tile: the
  // same operations in the same order, so the same results. Keys at or past
  // klim(q) = min(N, q + 1) of the lane's query get probability 0 and stay out
  // of the row maximum; 32-key blocks no query of the wave sees are skipped
  // whole.
  auto diag_tile = [&](int j, auto r_) __attribute__((always_inline)) {
    const unsigned char* Ks = k_base(r_);
    const unsigned char* Vs = v_base(r_);
    auto klim = [&](int q) { return min(N, q + 1); };
    int kvalid[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) kvalid[qb] = klim(qw0 + qb * 32 + l32) - j * S::BC;
    const int kbv = min(KB, max(1, (klim(qw0 + 32 * QB - 1) - j * S::BC + 31) >> 5));
    f32x16 sacc[QB][KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sacc[qb][kb] = f32x16{};
      if (kb >= kbv) continue;
#pragma unroll
      for (int cc = 0; cc < NCC; ++cc) {
        const u32x4 a = lds_read_b128(Ks, kb * 32 * S::ROWB + koff[cc]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sacc[qb][kb] = E::mfma(a, qf[qb][cc], sacc[qb][kb]);
      }
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if (kb >= kbv) continue;
        const int key = kb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          if (key >= kvalid[qb]) sacc[qb][kb][e] = -INFINITY;
      }
    float mnew[QB];
    bool need[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = sacc[qb][0][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if (kb >= kbv) continue;
#pragma unroll
        for (int e = (kb == 0 ? 1 : 0); e < 16; e += 2)
          mx = (e + 1 < 16) ? fmax3(mx, sacc[qb][kb][e], sacc[qb][kb][e + 1]) : fmax2(mx, sacc[qb][kb][e]);
      }
      mx = halves_max(mx) * c;
      mnew[qb] = fmaxf(m_run[qb], mx);
      need[qb] = mnew[qb] > m_run[qb] + kRescaleSlack;
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (__builtin_amdgcn_ballot_w64(need[qb])) {
        const float alpha = mnew[qb] == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[qb] - mnew[qb]);
        m_run[qb] = mnew[qb];
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[qb][db] *= alpha;
      }
    }
    u32x4 pd[QB][KB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float nm = -m_run[qb];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          if (kb >= kbv) continue;
          float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[qb][kb][e], c, nm));
          float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[qb][kb][e + 1], c, nm));
          const int key = kb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
          if (key >= kvalid[qb]) p0 = 0.f;
          if (key + 1 >= kvalid[qb]) p1 = 0.f;
          const uint32_t w = E::pack(p0, p1);
          pd[qb][kb][e >> 3][(e >> 1) & 3] = w;
          l_run[qb] = E::sum_pair(w, l_run[qb]);
        }
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          if (kb >= kbv) continue;
          const int rows = (kb * 32 + c2 * 16) * S::ROWB - VBIAS;
          const u32x4 a = cat(lds_read_tr16_b64(Vs, rows + voff[0][db]), lds_read_tr16_b64(Vs, rows + voff[1][db]));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = E::mfma(a, pd[qb][kb][c2], oacc[qb][db]);
        }
  };

  // Prologue: tiles 0 .. 2 resident, S of unit (0, 0).
  static_for<0, 3>([&](auto r_) __attribute__((always_inline)) {
    if (decltype(r_)::value < nt_dma) dma_tile(decltype(r_)::value, r_);
  });
  wait_vmem_below<0>();
  __syncthreads();
  if (nt > 0) {
    s_only(IntC<0>{}, IntC<0>{}, sa);
    tile(0, IntC<0>{}, BoolC<true>{}, BoolC<false>{});
    // Tiles 1 .. nt - 1, four per iteration (ring slots 1, 2, 3, 0), then the
    // rest. The last tile's last unit also computes S^T of tile nt, from the
    // slot it would occupy (tile nt - 4 without the mask, nt >= 4, no copy in
    // flight; the first diagonal tile under the causal mask, landed); the
    // result is never used. This keeps one tile body.
    int j = 1;
    for (; j + 4 <= nt; j += 4) {
      tile(j, IntC<1>{}, BoolC<false>{}, BoolC<false>{});
      tile(j + 1, IntC<2>{}, BoolC<false>{}, BoolC<false>{});
      tile(j + 2, IntC<3>{}, BoolC<false>{}, BoolC<false>{});
      tile(j + 3, IntC<0>{}, BoolC<false>{}, BoolC<false>{});
    }
    if (j < nt) tile(j, IntC<1>{}, BoolC<false>{}, BoolC<false>{});
    if (j + 1 < nt) tile(j + 1, IntC<2>{}, BoolC<false>{}, BoolC<false>{});
    if (j + 2 < nt) tile(j + 2, IntC<3>{}, BoolC<false>{}, BoolC<false>{});
    // P V of the last unit (tile nt - 1; query block 1 with two blocks, P^T in
    // pa; with one block, pa or pb by the tile's parity).
    constexpr int QL = QB - 1;
    switch ((nt - 1) % NS) {
      case 0: pv_only(IntC<0>{}, IntC<QL>{}, pa); break;
      case 1: pv_only(IntC<1>{}, IntC<QL>{}, QB == 2 ? pa : pb); break;
      case 2: pv_only(IntC<2>{}, IntC<QL>{}, pa); break;
      default: pv_only(IntC<3>{}, IntC<QL>{}, QB == 2 ? pa : pb); break;
    }
  }

  if constexpr (CAUSAL) {
    // The diagonal tiles nt .. nt_dma - 1, one at a time. Copies are issued in
    // tile order, and before tile j at most tiles j + 1 and j + 2 may still
    // be in flight; after the barrier every wave is done with tile j - 1,
    // whose slot takes tile j + 3.
    const int nvis_w = (qw0 + 32 * QB + S::BC - 1) / S::BC;  // tiles holding a key this wave's last query sees
    for (int j = nt; j < nt_dma; ++j) {
      const int ahead = min(2, nt_dma - 1 - j);
      if (ahead >= 2)
        wait_vmem_below<2 * PER>();
      else if (ahead == 1)
        wait_vmem_below<PER>();
      else
        wait_vmem_below<0>();
      __syncthreads();
      static_for<0, NS>([&](auto r_) __attribute__((always_inline)) {
        if (j + 3 < nt_dma && (j + 3) % NS == decltype(r_)::value) dma_tile(j + 3, r_);
      });
      if (j < nvis_w) {
        static_for<0, NS>([&](auto r_) __attribute__((always_inline)) {
          if (j % NS == decltype(r_)::value) diag_tile(j, r_);
        });
      }
    }
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = halves_sum(l_run[qb]);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const int q = qw0 + qb * 32 + l32;
    if (q < N) {
      uint16_t* orow = O + head_off(so, bh, H) + q * so.n;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x16& a = oacc[qb][db];
          u32x2 w = {E::pack(a[4 * jj] * inv, a[4 * jj + 1] * inv), E::pack(a[4 * jj + 2] * inv, a[4 * jj + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * jj + 4 * h) = w;
        }
      if (h == 0) LSE[(size_t)bh * N + q] = lt > 0.f ? (m_run[qb] + log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

// ------------------------------------------------------------------------
// fp32 forward: same method in fp32 storage and fp32 arithmetic (vector
// ALU). One workgroup = 256 threads for 8 query rows; thread (r, t) with
// r = tid / 32, t = tid % 32 scores keys t and t + 32 of each 64-key tile for
// query row r and owns output columns [t*D/32, (t+1)*D/32). Few rows per
// workgroup spread a short sequence over many CUs: one head of 196 rows runs
// as 25 workgroups, each with a quarter of the serial work per thread that 32
// rows per workgroup gave.
// ------------------------------------------------------------------------
constexpr int kF32BR = 8;
#ifndef FWD_F32_SPLIT
#define FWD_F32_SPLIT 1
#endif
constexpr int kBC = 64;  // keys per K/V tile of the fp32 kernel

// PF: the loads of the next K/V tile are issued before the current tile's
// arithmetic (registers for one more tile). For grids too small to fill the
// chip the tile loop is a chain of load latencies: one fp32 head, N=196, d=64
// 11.6-11.7 -> 10.7 us. On full grids the extra registers cost occupancy
// (d=64 +2 %, d=96 and 128 twice the time), so there each tile is loaded
// when it is needed.
template <int D, bool PF>
__global__ __launch_bounds__(256) void fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                      const float* __restrict__ V, float* __restrict__ O,
                                                      float* __restrict__ LSE, int N, int n_qblk, float scale) {
  // K rows padded to D + 4 floats and P rows to kBC + 4: 16-byte aligned rows
  // for 16-byte LDS reads. The 32 threads of a row read 32 consecutive keys'
  // rows (row offsets 4 banks apart: conflict-free in 16-lane quarters) and
  // consecutive output columns of V; rows of a wave share addresses.
  constexpr int KS = D + 4, PS = kBC + 4, DC = D / 32;
  __shared__ __attribute__((aligned(16))) float Ks[kBC * KS];
  __shared__ __attribute__((aligned(16))) float Vs[kBC * D];
  __shared__ __attribute__((aligned(16))) float Ps[kF32BR * PS];

  const int tid = threadIdx.x;
  const int bh = blockIdx.x / n_qblk, qblk = blockIdx.x - bh * n_qblk;
  const size_t head = (size_t)bh * N * D;
  const int r = tid >> 5, t = tid & 31;
  const int q = qblk * kF32BR + r;

  float4 qv[D / 4];
#pragma unroll
  for (int i = 0; i < D / 4; ++i)
    qv[i] = (q < N) ? *reinterpret_cast<const float4*>(Q + head + (size_t)q * D + 4 * i) : make_float4(0.f, 0.f, 0.f, 0.f);

  float acc[DC];
#pragma unroll
  for (int i = 0; i < DC; ++i) acc[i] = 0.f;
  float m = -INFINITY, l = 0.f;

  // With PF, K and V of the next tile wait in registers (kn, vn) while the
  // current one is computed.
  constexpr int PT = kBC * D / 4 / 256;  // float4 of K (and of V) per thread and tile
  static_assert(PT * 256 == kBC * D / 4, "a tile splits evenly over the threads");
  float4 kn[PT], vn[PT];
  auto load_tile = [&](int j0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int idx = tid + 256 * u, kr = idx / (D / 4), c4 = idx - kr * (D / 4);
      kn[u] = vn[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j0 + kr < N) {
        kn[u] = *reinterpret_cast<const float4*>(K + head + (size_t)(j0 + kr) * D + 4 * c4);
        vn[u] = *reinterpret_cast<const float4*>(V + head + (size_t)(j0 + kr) * D + 4 * c4);
      }
    }
  };
  if constexpr (PF) load_tile(0);
  for (int j0 = 0; j0 < N; j0 += kBC) {
    __syncthreads();
    if constexpr (PF) {
#pragma unroll
      for (int u = 0; u < PT; ++u) {
        const int idx = tid + 256 * u, kr = idx / (D / 4), c4 = idx - kr * (D / 4);
        *reinterpret_cast<float4*>(Ks + kr * KS + 4 * c4) = kn[u];
        *reinterpret_cast<float4*>(Vs + kr * D + 4 * c4) = vn[u];
      }
    } else {
      for (int idx = tid; idx < kBC * D / 4; idx += 256) {
        const int kr = idx / (D / 4), c4 = idx - kr * (D / 4);
        float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
        if (j0 + kr < N) {
          kk = *reinterpret_cast<const float4*>(K + head + (size_t)(j0 + kr) * D + 4 * c4);
          vv = *reinterpret_cast<const float4*>(V + head + (size_t)(j0 + kr) * D + 4 * c4);
        }
        *reinterpret_cast<float4*>(Ks + kr * KS + 4 * c4) = kk;
        *reinterpret_cast<float4*>(Vs + kr * D + 4 * c4) = vv;
      }
    }
    __syncthreads();
    if constexpr (PF) {
      if (j0 + kBC < N) load_tile(j0 + kBC);
    }

    // Scores of keys t and t + 32: two independent dot products, 4 dims per read.
    float s[2] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < D / 4; ++i)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float4 kv = *reinterpret_cast<const float4*>(Ks + (t + 32 * u) * KS + 4 * i);
        s[u] = fmaf(qv[i].x, kv.x, s[u]);
        s[u] = fmaf(qv[i].y, kv.y, s[u]);
        s[u] = fmaf(qv[i].z, kv.z, s[u]);
        s[u] = fmaf(qv[i].w, kv.w, s[u]);
      }
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      s[u] = (j0 + t + 32 * u < N) ? s[u] * scale : -INFINITY;
      mx = fmaxf(mx, s[u]);
    }
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    const float mnew = fmaxf(m, mx);
    const float alpha = expf(m - mnew);
    float rs = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float p = (j0 + t + 32 * u < N) ? expf(s[u] - mnew) : 0.f;
      rs += p;
      Ps[r * PS + t + 32 * u] = p;
    }
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) rs += __shfl_xor(rs, o);
    l = l * alpha + rs;
    m = mnew;
#pragma unroll
    for (int i = 0; i < DC; ++i) acc[i] *= alpha;
    __syncthreads();
    // O row r, columns t * DC ..: four keys' probabilities per read.
    for (int k4 = 0; k4 < kBC; k4 += 4) {
      const float4 p4 = *reinterpret_cast<const float4*>(Ps + r * PS + k4);
      const float pk[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int i = 0; i < DC; ++i) acc[i] = fmaf(pk[e], Vs[(k4 + e) * D + t * DC + i], acc[i]);
    }
  }
  if (q < N) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int i = 0; i < DC; ++i) O[head + (size_t)q * D + t * DC + i] = acc[i] * inv;
    if (t == 0) LSE[(size_t)bh * N + q] = m + logf(l);
  }
}

// fp32 forward for grids too small to fill the chip (one head of the ViT
// shape: 25 workgroups of kF32BR rows): there the time is the chain of key
// tiles each row walks through. Here the four waves of a workgroup take the
// same kF32SR rows and every fourth 64-key tile each (wave g: tiles g, g + 4,
// ...), each keeping its own running maximum, normaliser and partial output
// (§3, online-softmax bullet, applied per wave); at the end wave 0 merges the
// four partial states by the same rescaling. For 196 keys every wave walks one
// tile. All waves run the same number of iterations (a wave whose tile lies
// past N masks every key), so the workgroup barriers stay uniform. The
// launcher uses it for rows of at most four tiles.
constexpr int kF32SR = 2;
template <int D>
__global__ __launch_bounds__(256) void fwd_f32_split_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                            const float* __restrict__ V, float* __restrict__ O,
                                                            float* __restrict__ LSE, int N, int n_qblk, float scale) {
  static_assert(D == 32 || D == 64, "one wave loads a tile; LDS holds four");
  constexpr int KG = 4, KS = D + 4, PS = kBC + 4, DC = D / 32;
  constexpr int PT = kBC * D / 4 / 64;  // float4 of K (and of V) per lane and tile
  __shared__ __attribute__((aligned(16))) float Ks[KG][kBC * KS];
  __shared__ __attribute__((aligned(16))) float Vs[KG][kBC * D];
  __shared__ __attribute__((aligned(16))) float Ps[KG][kF32SR * PS];

  const int tid = threadIdx.x, g = tid >> 6, lane = tid & 63;
  const int r = lane >> 5, t = lane & 31;
  const int bh = blockIdx.x / n_qblk, qblk = blockIdx.x - bh * n_qblk;
  const size_t head = (size_t)bh * N * D;
  const int q = qblk * kF32SR + r;

  float4 qv[D / 4];
#pragma unroll
  for (int i = 0; i < D / 4; ++i)
    qv[i] = (q < N) ? *reinterpret_cast<const float4*>(Q + head + (size_t)q * D + 4 * i) : make_float4(0.f, 0.f, 0.f, 0.f);

  float acc[DC];
#pragma unroll
  for (int i = 0; i < DC; ++i) acc[i] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int n_tiles = (N + kBC - 1) / kBC, n_iter = (n_tiles + KG - 1) / KG;
  for (int it = 0; it < n_iter; ++it) {
    const int j0 = (it * KG + g) * kBC;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int idx = lane + 64 * u, kr = idx / (D / 4), c4 = idx - kr * (D / 4);
      float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
      if (j0 + kr < N) {
        kk = *reinterpret_cast<const float4*>(K + head + (size_t)(j0 + kr) * D + 4 * c4);
        vv = *reinterpret_cast<const float4*>(V + head + (size_t)(j0 + kr) * D + 4 * c4);
      }
      *reinterpret_cast<float4*>(&Ks[g][kr * KS + 4 * c4]) = kk;
      *reinterpret_cast<float4*>(&Vs[g][kr * D + 4 * c4]) = vv;
    }
    __syncthreads();

    // Scores of keys t and t + 32 of this wave's tile.
    float s[2] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < D / 4; ++i)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float4 kv = *reinterpret_cast<const float4*>(&Ks[g][(t + 32 * u) * KS + 4 * i]);
        s[u] = fmaf(qv[i].x, kv.x, s[u]);
        s[u] = fmaf(qv[i].y, kv.y, s[u]);
        s[u] = fmaf(qv[i].z, kv.z, s[u]);
        s[u] = fmaf(qv[i].w, kv.w, s[u]);
      }
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      s[u] = (j0 + t + 32 * u < N) ? s[u] * scale : -INFINITY;
      mx = fmaxf(mx, s[u]);
    }
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    const float mnew = fmaxf(m, mx);
    // A wave that has seen no key yet keeps m = -inf (and l = 0, acc = 0).
    const float alpha = mnew == -INFINITY ? 1.f : expf(m - mnew);
    float rs = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float p = (j0 + t + 32 * u < N) ? expf(s[u] - mnew) : 0.f;
      rs += p;
      Ps[g][r * PS + t + 32 * u] = p;
    }
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) rs += __shfl_xor(rs, o);
    l = l * alpha + rs;
    m = mnew;
#pragma unroll
    for (int i = 0; i < DC; ++i) acc[i] *= alpha;
    __syncthreads();
    for (int k4 = 0; k4 < kBC; k4 += 4) {
      const float4 p4 = *reinterpret_cast<const float4*>(&Ps[g][r * PS + k4]);
      const float pk[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int i = 0; i < DC; ++i) acc[i] = fmaf(pk[e], Vs[g][(k4 + e) * D + t * DC + i], acc[i]);
    }
  }

  // Merge: waves 1..3 leave (m, l, acc) in LDS (over their K tiles), wave 0
  // rescales each partial state to the common maximum and adds.
  __syncthreads();
  float* part = &Ks[0][0];  // [KG][kF32SR][32][2 + DC]
  constexpr int PW = 2 + DC;
  if (g > 0) {
    float* e = part + ((g * kF32SR + r) * 32 + t) * PW;
    e[0] = m;
    e[1] = l;
#pragma unroll
    for (int i = 0; i < DC; ++i) e[2 + i] = acc[i];
  }
  __syncthreads();
  if (g > 0) return;
  float mt = m;
#pragma unroll
  for (int o = 1; o < KG; ++o) mt = fmaxf(mt, part[((o * kF32SR + r) * 32 + t) * PW]);
  const float a0 = m == -INFINITY ? 0.f : expf(m - mt);
  float lt = l * a0;
#pragma unroll
  for (int i = 0; i < DC; ++i) acc[i] *= a0;
#pragma unroll
  for (int o = 1; o < KG; ++o) {
    const float* e = part + ((o * kF32SR + r) * 32 + t) * PW;
    const float a = e[0] == -INFINITY ? 0.f : expf(e[0] - mt);
    lt = fmaf(e[1], a, lt);
#pragma unroll
    for (int i = 0; i < DC; ++i) acc[i] = fmaf(e[2 + i], a, acc[i]);
  }
  if (q < N) {
    const float inv = 1.0f / lt;
#pragma unroll
    for (int i = 0; i < DC; ++i) O[head + (size_t)q * D + t * DC + i] = acc[i] * inv;
    if (t == 0) LSE[(size_t)bh * N + q] = mt + logf(lt);
  }
}

}  // namespace

template <class E, int D, int QB, int KB>
static hipError_t launch_fwd_pp(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                                int B, int H, int N, float scale, Strides sq, Strides so, hipStream_t stream) {
  using S = FwdShape<D, QB, KB, kPPRing, kPPWaves>;
  const int n_qblk = (N + S::BR - 1) / S::BR;
  const int total = n_qblk * B * H;
  const float c = fabsf(scale) * kLog2e;
  const uint32_t qsign = scale < 0.f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((fwd_pp_kernel<E, D, QB, KB>), dim3(total), dim3(S::THREADS), 0, stream, q, k, v, o, lse, N,
                     n_qblk, total, c, qsign, H, sq, so);
  return hipGetLastError();
}

template <class E, int D, int QB, int WAVES, bool CAUSAL>
static hipError_t launch_fwd_sp(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                                int B, int H, int N, float scale, Strides sq, Strides so, hipStream_t stream) {
  using S = FwdShape<D, QB, 2, kSPRing, WAVES>;
  const int n_qblk = (N + S::BR - 1) / S::BR;
  const int total = n_qblk * B * H;
  const float c = fabsf(scale) * kLog2e;
  const uint32_t qsign = scale < 0.f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((fwd_sp_kernel<E, D, QB, WAVES, CAUSAL>), dim3(total), dim3(S::THREADS), 0, stream, q, k, v, o, lse, N,
                     n_qblk, total, c, qsign, H, sq, so);
  return hipGetLastError();
}

template <class E, int D, int QB, int KB, int NS, int WAVES>
static hipError_t launch_fwd_t(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                                    float* lse, int B, int H, int N, float scale, int causal, const int* kv_len,
                                    Strides sq, Strides so, hipStream_t stream) {
  using S = FwdShape<D, QB, KB, NS, WAVES>;
  const int n_qblk = (N + S::BR - 1) / S::BR;
  const int total = n_qblk * B * H;
  const float c = fabsf(scale) * kLog2e;
  const uint32_t qsign = scale < 0.f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((fwd_kernel<E, D, QB, KB, NS, WAVES>), dim3(total), dim3(S::THREADS), 0, stream, q, k, v, o,
                     lse, N, n_qblk, total, c, qsign, kv_len, H, causal, sq, so);
  return hipGetLastError();
}

// Launch shapes per head dim (long rows: 8-wave workgroups, for d = 32 and 64
// only from FWD_LONG_N_SMALL_D keys on; short: 4-wave):
//   d = 32:  one 32-query block per wave, 128-key tiles (long) or two blocks and 64-key tiles (short);
//   d = 64:  FWD_QB64 / FWD_KB64 / FWD_NS64;
//   d = 96:  one query block, 128-key tiles (192-byte rows: 64-key tiles would not split evenly over the
//            DMA lanes);
//   d = 128: FWD_QB128 / FWD_KB128 / FWD_NS128.
template <class E>
static hipError_t launch_fwd_e(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                               int B, int H, int N, int d, float scale, int causal, const int* kv_len,
                               Strides sq, Strides so, hipStream_t stream) {
  const bool lng = N >= FWD_LONG_N;
  // d = 32 and 64 keep 4-wave workgroups (two per CU) up to FWD_LONG_N_SMALL_D
  // keys: their tiles are cheap to re-read from L2, and the finer grid
  // balances the causal triangle (measured at N = 4096: d = 64 -2.5 %, causal
  // -18 %; d = 32 -9 %, causal -17 %; at N = 16384, d = 64, 8 waves are 1.5 %
  // faster). d = 96 and 128 measured 18-24 % slower with 4 waves.
  const bool lng_small_d = N >= FWD_LONG_N_SMALL_D;
  // Rows without masks, whole 64-key tiles, d = 64: the software-pipelined forward.
  if (FWD_SP && d == 64 && !causal && !kv_len && N % 64 == 0 && N >= FWD_SP_MIN_N)
    return launch_fwd_sp<E, 64, 2, 4, false>(q, k, v, o, lse, B, H, N, scale, sq, so, stream);
  // Causal rows at d = 64: one query block per wave (128-query workgroups, which balance the diagonal as
  // fwd_kernel's do), from FWD_SP64_CAUSAL_MIN_N keys.
  if (FWD_SP && FWD_SP64_CAUSAL && d == 64 && causal && !kv_len && N % 64 == 0 && N >= FWD_SP64_CAUSAL_MIN_N)
    return launch_fwd_sp<E, 64, 1, 4, true>(q, k, v, o, lse, B, H, N, scale, sq, so, stream);
  // d = 128: one query block per wave, 8 waves sharing the ring (128 KB of LDS, one workgroup per CU). With the
  // causal mask (FWD_SP_CAUSAL) the kernel takes the tiles a workgroup's queries see in full and finishes with
  // the diagonal tiles (at d = 64 the single-phase kernel's 128-query workgroups balance the diagonal better).
  if (FWD_SP128 && d == 128 && !kv_len && (!causal || FWD_SP_CAUSAL) && N % 64 == 0 && N >= FWD_SP128_MIN_N)
    return causal ? launch_fwd_sp<E, 128, 1, 8, true>(q, k, v, o, lse, B, H, N, scale, sq, so, stream)
                  : launch_fwd_sp<E, 128, 1, 8, false>(q, k, v, o, lse, B, H, N, scale, sq, so, stream);
  if (FWD_PINGPONG && lng && !causal && !kv_len) {
#if FWD_PP_D64
    if (d == 64)
      return launch_fwd_pp<E, 64, FWD_PP_QB64, FWD_PP_KB64>(q, k, v, o, lse, B, H, N, scale, sq, so, stream);
#endif
    if (d == 128)
      return launch_fwd_pp<E, 128, FWD_PP_QB128, FWD_PP_KB128>(q, k, v, o, lse, B, H, N, scale, sq, so, stream);
  }
#define ATTN_FWD(D, QB, KB, NS, W) \
  launch_fwd_t<E, D, QB, KB, NS, W>(q, k, v, o, lse, B, H, N, scale, causal, kv_len, sq, so, stream)
  switch (d) {
    case 32:
      return lng_small_d ? ATTN_FWD(32, 1, 4, 2, FWD_WAVES_LONG)
                         : (lng ? ATTN_FWD(32, 1, 4, 2, 4) : ATTN_FWD(32, 2, 2, FWD_NS_SHORT, 4));
    case 64:
      return lng_small_d ? ATTN_FWD(64, FWD_QB64, FWD_KB64, FWD_NS64, FWD_WAVES_LONG)
                         : ATTN_FWD(64, FWD_QB64_SHORT, FWD_KB64, FWD_NS_SHORT, FWD_WAVES_SHORT64);
    case 96:
      return lng ? ATTN_FWD(96, 1, 4, 2, FWD_WAVES_LONG) : ATTN_FWD(96, 1, 4, 2, 4);
    default:
      return lng ? ATTN_FWD(128, FWD_QB128, FWD_KB128, FWD_NS128, FWD_WAVES_LONG)
                 : ATTN_FWD(128, FWD_QB128, FWD_KB128, FWD_NS_SHORT, 4);
  }
#undef ATTN_FWD
}

hipError_t launch_fwd_16(bool f16, const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse,
                         int B, int H, int N, int d, float scale, int causal, const int* kv_len, Strides sq, Strides so,
                         hipStream_t stream) {
  return f16 ? launch_fwd_e<F16>(q, k, v, o, lse, B, H, N, d, scale, causal, kv_len, sq, so, stream)
             : launch_fwd_e<Bf16>(q, k, v, o, lse, B, H, N, d, scale, causal, kv_len, sq, so, stream);
}

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N,
                          int d, float scale, hipStream_t stream) {
  const int n_qblk = (N + kF32BR - 1) / kF32BR;
  const int total = n_qblk * B * H;
  const bool pf = total < 256 && d <= 64;  // under one workgroup per CU: latency-bound
  // Rows of at most 4 tiles: the key-split kernel, one tile per wave (measured, B=1, H=1, N=196, d=64: 10.8 ->
  // 6.9 us per call). With more tiles per wave it lost (N = 300: 9.7 -> 15.2 us; N = 700: 26 -> 42 us): it
  // has no prefetch, and its 2-row workgroups read every K/V tile four times as often.
  if (pf && FWD_F32_SPLIT && N <= 4 * kBC) {
    const int n_sblk = (N + kF32SR - 1) / kF32SR;
    if (d == 32)
      hipLaunchKernelGGL((fwd_f32_split_kernel<32>), dim3(n_sblk * B * H), dim3(256), 0, stream, q, k, v, o, lse, N,
                         n_sblk, scale);
    else
      hipLaunchKernelGGL((fwd_f32_split_kernel<64>), dim3(n_sblk * B * H), dim3(256), 0, stream, q, k, v, o, lse, N,
                         n_sblk, scale);
    return hipGetLastError();
  }
#define ATTN_FWD_F32(D)                                                                                           \
  if (pf)                                                                                                         \
    hipLaunchKernelGGL((fwd_f32_kernel<D, D <= 64>), dim3(total), dim3(256), 0, stream, q, k, v, o, lse, N, n_qblk, \
                       scale);                                                                                    \
  else                                                                                                            \
    hipLaunchKernelGGL((fwd_f32_kernel<D, false>), dim3(total), dim3(256), 0, stream, q, k, v, o, lse, N, n_qblk, scale)
  switch (d) {
    case 32: ATTN_FWD_F32(32); break;
    case 64: ATTN_FWD_F32(64); break;
    case 96: ATTN_FWD_F32(96); break;
    default: ATTN_FWD_F32(128);
  }
#undef ATTN_FWD_F32
  return hipGetLastError();
}

}  // namespace attn
