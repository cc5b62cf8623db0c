// attn_api.hip - the extern "C" entry points of libattn.so (declared in
// include/attn.h): argument validation, head-dim dispatch and launch. Every
// check runs on the host before anything is enqueued, so a rejected call
// launches nothing and writes nothing.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/attn.h"
#include "attn_kernels.h"

namespace {

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;
};

Range span(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Shared shape checks. Returns ATTN_OK and the element counts, or an error code.
int check_shape(int B, int H, int N, int d, float scale, size_t* elems, size_t* rows) {
  if (B < 1 || H < 1 || N < 1) return ATTN_ERR_INVALID_ARG;
  if (!isfinite(scale)) return ATTN_ERR_INVALID_ARG;
  if (d != 32 && d != 64 && d != 96 && d != 128) return ATTN_ERR_UNSUPPORTED;
  // Kernels index within a head with 32-bit ints and launch one workgroup per
  // (head, row block) on a 1-D grid.
  const int64_t per_head = (int64_t)N * d;
  const int64_t heads = (int64_t)B * H;
  if (per_head > INT32_MAX / 2) return ATTN_ERR_UNSUPPORTED;
  if (heads * ((N + 31) / 32) > INT32_MAX / 2) return ATTN_ERR_UNSUPPORTED;
  *rows = (size_t)heads * (size_t)N;
  *elems = *rows * (size_t)d;
  return ATTN_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

// Strides of the tensor groups (q, k, v), (o, dO) and (dq, dk, dv) for a layout.
struct Layout {
  attn::Strides qkv, o, grad;
  bool packed;  // q, k, v (and dq, dk, dv) interleaved in one [B, N, 3, H, d] buffer
};

int make_layout(int layout, int B, int H, int N, int d, Layout* L) {
  const long long hd = (long long)H * d, nd = (long long)N * d;
  (void)B;
  switch (layout) {
    case ATTN_LAYOUT_BHND:
      L->qkv = attn::Strides{H * nd, nd, d};
      L->o = L->grad = L->qkv;
      L->packed = false;
      break;
    case ATTN_LAYOUT_BNHD:
      L->qkv = attn::Strides{N * hd, d, (int)hd};
      L->o = L->grad = L->qkv;
      L->packed = false;
      break;
    case ATTN_LAYOUT_QKV_PACKED:
      L->qkv = attn::Strides{3 * N * hd, d, (int)(3 * hd)};
      L->o = attn::Strides{N * hd, d, (int)hd};
      L->grad = L->qkv;
      L->packed = true;
      break;
    default:
      return ATTN_ERR_UNSUPPORTED;
  }
  // Rows of a head are addressed with 32-bit element offsets.
  if ((long long)N * L->qkv.n > INT32_MAX / 2) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

// For the packed layout: the second and third tensor sit H * d and 2 H * d elements after the first.
bool packed_trio(const void* a, const void* b, const void* c, size_t hd_bytes) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a);
  return reinterpret_cast<uintptr_t>(b) == x + hd_bytes && reinterpret_cast<uintptr_t>(c) == x + 2 * hd_bytes;
}

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, B/H/N < 1, non-finite scale, causal not 0 or 1, or overlapping buffers)";
    case ATTN_ERR_UNSUPPORTED: return "unsupported (d_k must be 32, 64, 96 or 128, dtype must be known, sizes must fit 32-bit per-head indexing)";
    case ATTN_ERR_WORKSPACE: return "workspace missing or smaller than attn_bwd_workspace_bytes()";
    case ATTN_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

int attn_fwd_ex(int dtype, int layout, const void* q, const void* k, const void* v, void* o, float* lse, int B,
                int H, int N, int d_k, float scale, int causal, const int* kv_len, void* stream) {
  size_t E = 0, R = 0;
  int st = check_shape(B, H, N, d_k, scale, &E, &R);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_F16) return ATTN_ERR_UNSUPPORTED;
  Layout L;
  if ((st = make_layout(layout, B, H, N, d_k, &L)) != ATTN_OK) return st;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return ATTN_ERR_INVALID_ARG;
  if (kv_len != nullptr && (reinterpret_cast<uintptr_t>(kv_len) & 3u) != 0) return ATTN_ERR_INVALID_ARG;
  if (L.packed && !packed_trio(q, k, v, (size_t)H * d_k * 2)) return ATTN_ERR_INVALID_ARG;
  // Extents: a packed q, k, v buffer is one 3 E element range starting at q.
  const Range rq = L.packed ? span(q, 3 * E * 2) : span(q, E * 2);
  const Range rk = L.packed ? rq : span(k, E * 2), rv = L.packed ? rq : span(v, E * 2);
  const Range ro = span(o, E * 2), rl = span(lse, R * 4);
  if (overlap(ro, rq) || overlap(ro, rk) || overlap(ro, rv) || overlap(ro, rl)) return ATTN_ERR_INVALID_ARG;
  if (overlap(rl, rq) || overlap(rl, rk) || overlap(rl, rv)) return ATTN_ERR_INVALID_ARG;
  if (kv_len != nullptr) {
    const Range rkv = span(kv_len, (size_t)B * 4);
    if (overlap(rkv, ro) || overlap(rkv, rl)) return ATTN_ERR_INVALID_ARG;
  }
  return from_hip(attn::launch_fwd_16(dtype == ATTN_DTYPE_F16, static_cast<const uint16_t*>(q),
                                      static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                                      static_cast<uint16_t*>(o), lse, B, H, N, d_k, scale, causal, kv_len, L.qkv, L.o,
                                      static_cast<hipStream_t>(stream)));
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d_k,
             float scale, void* stream) {
  return attn_fwd_ex(ATTN_DTYPE_BF16, ATTN_LAYOUT_BHND, q, k, v, o, lse, B, H, N, d_k, scale, 0, nullptr, stream);
}

int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N, int d_k,
                 float scale, void* stream) {
  size_t E = 0, R = 0;
  const int st = check_shape(B, H, N, d_k, scale, &E, &R);
  if (st != ATTN_OK) return st;
  // The fp32 forward launches one workgroup per 8 rows of a head.
  if ((int64_t)B * H * ((N + 7) / 8) > INT32_MAX / 2) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return ATTN_ERR_INVALID_ARG;
  const Range rq = span(q, E * 4), rk = span(k, E * 4), rv = span(v, E * 4), ro = span(o, E * 4), rl = span(lse, R * 4);
  if (overlap(ro, rq) || overlap(ro, rk) || overlap(ro, rv) || overlap(ro, rl)) return ATTN_ERR_INVALID_ARG;
  if (overlap(rl, rq) || overlap(rl, rk) || overlap(rl, rv)) return ATTN_ERR_INVALID_ARG;
  return from_hip(attn::launch_fwd_f32(q, k, v, o, lse, B, H, N, d_k, scale, static_cast<hipStream_t>(stream)));
}

size_t attn_bwd_workspace_bytes(int B, int H, int N, int d_k) {
  size_t E = 0, R = 0;
  if (check_shape(B, H, N, d_k, 1.0f, &E, &R) != ATTN_OK) return 0;
  return attn::bwd_workspace_bytes(B, H, N, d_k);
}

namespace {

// dtype -1 stands for float32 storage (attn_bwd_f32, contiguous layout only).
// with_ws false: the workspace is the library's own scratch array (checked by
// the caller), so only the other arguments are validated here.
int bwd_checks(int dtype, int layout, const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d_k, float scale, int causal,
               const int* kv_len, void* workspace, size_t workspace_bytes, Layout* L, bool with_ws = true) {
  size_t E = 0, R = 0;
  int st = check_shape(B, H, N, d_k, scale, &E, &R);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_F16 && dtype != -1) return ATTN_ERR_UNSUPPORTED;
  if ((st = make_layout(layout, B, H, N, d_k, L)) != ATTN_OK) return st;
  const size_t esz = dtype == -1 ? 4 : 2;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID_ARG;
  if (kv_len != nullptr && (reinterpret_cast<uintptr_t>(kv_len) & 3u) != 0) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) || !aligned16(dO) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return ATTN_ERR_INVALID_ARG;
  const size_t hd_bytes = (size_t)H * d_k * esz;
  if (L->packed && (!packed_trio(q, k, v, hd_bytes) || !packed_trio(dq, dk, dv, hd_bytes))) return ATTN_ERR_INVALID_ARG;
  const size_t need = attn::bwd_workspace_bytes(B, H, N, d_k);
  if (with_ws) {
    if (workspace == nullptr || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return ATTN_ERR_INVALID_ARG;
  }
  // Extents: packed q, k, v (and dq, dk, dv) are one 3 E element buffer each.
  const size_t tb = E * esz, pb = L->packed ? 3 * tb : tb;
  const Range ins[6] = {span(q, pb), L->packed ? span(q, pb) : span(k, tb), L->packed ? span(q, pb) : span(v, tb),
                        span(o, tb), span(dO, tb), span(lse, R * 4)};
  const Range outs[4] = {span(dq, pb), L->packed ? span(dq, pb) : span(dk, tb), L->packed ? span(dq, pb) : span(dv, tb),
                         span(workspace, need)};
  const int n_out = with_ws ? 4 : 3;
  for (int a = 0; a < n_out; ++a) {
    for (int b = 0; b < 6; ++b)
      if (overlap(outs[a], ins[b])) return ATTN_ERR_INVALID_ARG;
    for (int b = a + 1; b < n_out; ++b)  // packed dq, dk, dv interleave by construction
      if (!(L->packed && b < 3) && overlap(outs[a], outs[b])) return ATTN_ERR_INVALID_ARG;
    if (kv_len != nullptr && overlap(outs[a], span(kv_len, (size_t)B * 4))) return ATTN_ERR_INVALID_ARG;
  }
  return ATTN_OK;
}

int bwd_launch(int dtype, int stage, const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d_k, float scale, int causal,
               const int* kv_len, const Layout& L, void* workspace, void* stream) {
  const attn::Strides st[4] = {L.qkv, L.o, L.o, L.grad};
  return from_hip(attn::launch_bwd_16_stage(
      dtype == ATTN_DTYPE_F16, stage, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(o), lse, static_cast<const uint16_t*>(dO),
      static_cast<uint16_t*>(dq), static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), B, H, N, d_k, scale, causal,
      kv_len, st, workspace, static_cast<hipStream_t>(stream)));
}

// The backward's workspace for callers that cannot allocate (attn_bwd_ex_noalloc):
// a file-scope device array, one copy per GPU, held until the process ends.
// In host code `scratch` names a host-side stand-in, never the device memory:
// kernels get the per-device address from hipGetSymbolAddress below.
constexpr size_t kScratchBytes = size_t(16) << 20;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device `stream` belongs to, looked up once
// per device with that device current.
int scratch_for_stream(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess) return ATTN_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return ATTN_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return ATTN_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return ATTN_ERR_HIP;
    if (e != hipSuccess || p == nullptr) return ATTN_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

int attn_bwd_f32(const float* q, const float* k, const float* v, const float* o, const float* lse, const float* dO,
                 float* dq, float* dk, float* dv, int B, int H, int N, int d_k, float scale, void* workspace,
                 size_t workspace_bytes, void* stream) {
  Layout L;
  const int st = bwd_checks(-1, ATTN_LAYOUT_BHND, q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d_k, scale, 0, nullptr,
                            workspace, workspace_bytes, &L);
  if (st != ATTN_OK) return st;
  for (int stage = 0; stage < 3; ++stage) {
    const int r = from_hip(attn::launch_bwd_f32_stage(stage, q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d_k, scale,
                                                      workspace, static_cast<hipStream_t>(stream)));
    if (r != ATTN_OK) return r;
  }
  return ATTN_OK;
}

int attn_bwd_ex(int dtype, int layout, const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d_k, float scale, int causal,
                const int* kv_len, void* workspace, size_t workspace_bytes, void* stream) {
  // The 16-bit types only (bwd_checks also serves attn_bwd_f32, with dtype -1).
  if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_F16) return ATTN_ERR_UNSUPPORTED;
  Layout L;
  const int st = bwd_checks(dtype, layout, q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d_k, scale, causal, kv_len,
                            workspace, workspace_bytes, &L);
  if (st != ATTN_OK) return st;
  const int stages_fused[2] = {0, 3}, stages[3] = {0, 1, 2};
  const bool fuse = attn::bwd_can_fuse(B, H, N, d_k);
  for (int i = 0; i < (fuse ? 2 : 3); ++i) {
    const int r = bwd_launch(dtype, fuse ? stages_fused[i] : stages[i], q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d_k,
                             scale, causal, kv_len, L, workspace, stream);
    if (r != ATTN_OK) return r;
  }
  return ATTN_OK;
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO, void* dq,
             void* dk, void* dv, int B, int H, int N, int d_k, float scale, void* workspace, size_t workspace_bytes,
             void* stream) {
  return attn_bwd_ex(ATTN_DTYPE_BF16, ATTN_LAYOUT_BHND, q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d_k, scale, 0,
                     nullptr, workspace, workspace_bytes, stream);
}

int attn_bwd_ex_noalloc(int dtype, int layout, const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d_k,
                        float scale, int causal, const int* kv_len, void* stream) {
  if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_F16) return ATTN_ERR_UNSUPPORTED;
  Layout L;
  int st = bwd_checks(dtype, layout, q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d_k, scale, causal, kv_len, nullptr, 0,
                      &L, false);
  if (st != ATTN_OK) return st;
  if (attn::bwd_workspace_bytes(B, H, N, d_k) > kScratchBytes) return ATTN_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_for_stream(static_cast<hipStream_t>(stream), &ws)) != ATTN_OK) return st;
  // The same launches as attn_bwd_ex; stage 0 writes every workspace element the later stages read.
  const int stages_fused[2] = {0, 3}, stages[3] = {0, 1, 2};
  const bool fuse = attn::bwd_can_fuse(B, H, N, d_k);
  for (int i = 0; i < (fuse ? 2 : 3); ++i) {
    const int r = bwd_launch(dtype, fuse ? stages_fused[i] : stages[i], q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d_k,
                             scale, causal, kv_len, L, ws, stream);
    if (r != ATTN_OK) return r;
  }
  return ATTN_OK;
}

int attn_bwd_stage(int stage, int dtype, int layout, const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d_k,
                   float scale, int causal, const int* kv_len, void* workspace, size_t workspace_bytes,
                   void* stream) {
  if (stage < 0 || stage > 3) return ATTN_ERR_INVALID_ARG;
  if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_F16) return ATTN_ERR_UNSUPPORTED;
  Layout L;
  const int st = bwd_checks(dtype, layout, q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d_k, scale, causal, kv_len,
                            workspace, workspace_bytes, &L);
  if (st != ATTN_OK) return st;
  if (stage == 3 && !attn::bwd_can_fuse(B, H, N, d_k)) {  // stages 1 and 2 as separate launches
    const int r = bwd_launch(dtype, 1, q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d_k, scale, causal, kv_len, L,
                             workspace, stream);
    if (r != ATTN_OK) return r;
    stage = 2;
  }
  return bwd_launch(dtype, stage, q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d_k, scale, causal, kv_len, L, workspace,
                    stream);
}

// Shape checks of the projection: returns ATTN_OK and the token count and
// output width 3 H d_k, or an error code.
static int proj_shape(int dtype, int B, int N, int D, int H, int d_k, long* tokens, int* hd3) {
  if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_F16) return ATTN_ERR_UNSUPPORTED;
  if (B < 1 || N < 1 || D < 1 || H < 1 || d_k < 1) return ATTN_ERR_INVALID_ARG;
  const int64_t t = (int64_t)B * N, hd = (int64_t)H * d_k;
  if (D % 8 != 0 || hd % 8 != 0) return ATTN_ERR_UNSUPPORTED;
  if (t >= (int64_t)1 << 30 || 3 * hd > INT32_MAX / 2 || D > INT32_MAX / 2) return ATTN_ERR_UNSUPPORTED;
  *tokens = (long)t;
  *hd3 = (int)(3 * hd);
  return ATTN_OK;
}

int attn_qkv_proj(int dtype, const void* x, const void* w, void* qkv, int B, int N, int D, int H, int d_k,
                  void* stream) {
  long T = 0;
  int HD3 = 0;
  int st = proj_shape(dtype, B, N, D, H, d_k, &T, &HD3);
  if (st != ATTN_OK) return st;
  if (!aligned16(x) || !aligned16(w) || !aligned16(qkv)) return ATTN_ERR_INVALID_ARG;
  const Range rx = span(x, (size_t)T * D * 2), rw = span(w, (size_t)D * HD3 * 2), ry = span(qkv, (size_t)T * HD3 * 2);
  if (overlap(ry, rx) || overlap(ry, rw)) return ATTN_ERR_INVALID_ARG;
  return from_hip(attn::launch_proj_fwd(dtype == ATTN_DTYPE_F16, static_cast<const uint16_t*>(x),
                                        static_cast<const uint16_t*>(w), static_cast<uint16_t*>(qkv), T, D, HD3,
                                        static_cast<hipStream_t>(stream)));
}

size_t attn_qkv_proj_bwd_workspace_bytes(int B, int N, int D, int H, int d_k) {
  long T = 0;
  int HD3 = 0;
  if (proj_shape(ATTN_DTYPE_BF16, B, N, D, H, d_k, &T, &HD3) != ATTN_OK) return 0;
  return attn::proj_bwd_workspace_bytes(T, D, HD3);
}

int attn_qkv_proj_bwd(int dtype, const void* x, const void* w, const void* dqkv, void* dx, void* dw, int B, int N,
                      int D, int H, int d_k, void* workspace, size_t workspace_bytes, void* stream) {
  long T = 0;
  int HD3 = 0;
  int st = proj_shape(dtype, B, N, D, H, d_k, &T, &HD3);
  if (st != ATTN_OK) return st;
  if (!aligned16(x) || !aligned16(w) || !aligned16(dqkv) || !aligned16(dx) || !aligned16(dw))
    return ATTN_ERR_INVALID_ARG;
  const size_t need = attn::proj_bwd_workspace_bytes(T, D, HD3);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return ATTN_ERR_INVALID_ARG;
  const Range rx = span(x, (size_t)T * D * 2), rw = span(w, (size_t)D * HD3 * 2);
  const Range rg = span(dqkv, (size_t)T * HD3 * 2), rdx = span(dx, (size_t)T * D * 2), rdw = span(dw, (size_t)D * HD3 * 2);
  if (overlap(rdx, rdw)) return ATTN_ERR_INVALID_ARG;
  for (const Range& o : {rdx, rdw})
    if (overlap(o, rx) || overlap(o, rw) || overlap(o, rg)) return ATTN_ERR_INVALID_ARG;
  if (need > 0) {
    const Range rws = span(workspace, need);
    for (const Range& o : {rx, rw, rg, rdx, rdw})
      if (overlap(rws, o)) return ATTN_ERR_INVALID_ARG;
  }
  return from_hip(attn::launch_proj_bwd(dtype == ATTN_DTYPE_F16, static_cast<const uint16_t*>(x),
                                        static_cast<const uint16_t*>(w), static_cast<const uint16_t*>(dqkv),
                                        static_cast<uint16_t*>(dx), static_cast<uint16_t*>(dw), T, D, HD3,
                                        need > 0 ? workspace : nullptr, static_cast<hipStream_t>(stream)));
}

int attn_bwd_fused(int B, int H, int N, int d_k) {
  size_t E = 0, R = 0;
  if (check_shape(B, H, N, d_k, 1.0f, &E, &R) != ATTN_OK) return 0;
  return attn::bwd_can_fuse(B, H, N, d_k) ? 1 : 0;
}

}  // extern "C"
