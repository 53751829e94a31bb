// Reverse pass of the fused attention forward with tangents, for gfx950.
//
// With cotangents G of O and Gd of dO (L = <G, O> + <Gd, dO>), the forward's
// intermediates per (query i, key j) -- P, the score tangent Sd = dS, and
// Pd = P (Sd - tlse) -- give
//   D    = Gd V^T                       (the cotangent of Pd)
//   r_i  = Gd_i . O_i                   (= sum_j D_ij P_ij)
//   dP   = G V^T + Gd dV^T + D (Sd - tlse) - r Sd
//   del_i = G_i . O_i + Gd_i . dO_i - tlse_i r_i   (= sum_j P_ij dP_ij)
//   Sbar  = P (dP - del)                cotangent of the scores
//   Sdbar = P (D - r)                   cotangent of the score tangents
//   dq  = scale (Sbar K + Sdbar dK)     dk  = scale (Sbar^T Q + Sdbar^T dQ)
//   dtq = scale Sdbar K                 dtk = scale Sdbar^T Q
//   dv  = P^T G + Pd^T Gd               dtv = P^T Gd
// which is the chain rule run backwards through the forward's steps (the
// float64 oracle runs those steps one at a time; the two agree to rounding).
// The N x N matrices are never stored: three kernels recompute them per tile.
//   rows: per query row r, del and -lse*log2(e) and tlse into the workspace;
//   dkv:  128 keys (of one K/V head) per work item, looping over 32-query
//         tiles (at d = 64 without a mask, one workgroup per CU walks
//         several items);
//   dq:   128 queries per workgroup, looping over 32-key tiles (large d = 64
//         grids: two workgroups per CU, without the software pipeline).
// Both tile kernels use the forward's MFMA layout (32x32x16 products, C
// registers rounded to 16 bits reused as B operands, transpose reads of the
// LDS tiles for the accumulating products). They depend only on the rows
// kernel, so the query side may run on a second stream beside the key side.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "jvpattn.h"
#include "jvpattn_bwd_launch.h"
#include "jvpattn_fwd_launch.h"
#include "jvpattn_internal.h"

namespace jvpattn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Running the query side beside the key side. The two kernels share only
// the rows kernel's output, so the query side may run on a second stream
// that waits for the rows kernel, and the caller's stream waits for it in
// turn: as the key side's workgroups finish, the query side's take their
// compute units, instead of starting only after the last key-side workgroup.
// The second stream and its two events are the library's, one set per
// device, created on first use and kept until the process ends; a mutex
// holds the record-wait-launch sequence together across host threads.
// Mode (jvpattn_bwd_set_overlap): -1 automatic, 0 one stream, 1 two streams.
// Automatic takes two streams where the key side alone would leave compute
// units idle: fewer key-side items (128-key blocks x K/V heads) than CUs;
// under a causal limit, fewer than two per CU (one item per workgroup, the
// first key blocks many times longer than the last; with two or more per
// workgroup the walking order pairs long with short ones); and at d = 128
// (the key side in two launches). Elsewhere the key side's workgroups end
// nearly together and a second kernel only takes CUs from its last items.
std::atomic<int> g_overlap{-1};

constexpr int kMaxSideDevices = 64;
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t rows = nullptr;   // recorded on the caller's stream after the rows kernel
  hipEvent_t done = nullptr;   // recorded on the side stream after the query side
};
std::mutex g_side_mu;
SideStream g_side[kMaxSideDevices];

// The side stream set of `dev` (g_side_mu held).
hipError_t side_stream(int dev, SideStream** out) {
  if (dev < 0 || dev >= kMaxSideDevices) return hipErrorInvalidDevice;
  SideStream& x = g_side[dev];
  if (!x.s) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    SideStream n;
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&n.s, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&n.rows, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&n.done, hipEventDisableTiming);
    if (cur >= 0 && cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) {
      if (n.done) (void)hipEventDestroy(n.done);
      if (n.rows) (void)hipEventDestroy(n.rows);
      if (n.s) (void)hipStreamDestroy(n.s);
      return e;
    }
    x = n;
  }
  *out = &x;
  return hipSuccess;
}

// Queue the reverse pass for arguments already validated; tmask: the
// additive mask's tangent the forward carried, or NULL.
// may_fork: the query side may run on the library's second stream.
int bwd_launch(const jvpattn_params* p, const FwdSizes& sz, const void* q, const void* k, const void* v,
               const void* tq, const void* tk, const void* tv, const void* mask, const void* tmask,
               const void* o, const void* to, const float* lse, const float* tlse, const void* go,
               const void* gto, void* dq, void* dk, void* dv, void* dtq, void* dtk, void* dtv, void* workspace,
               void* stream, bool may_fork) {
  if (sz.rows_q == 0 && sz.rows_k == 0) return JVPATTN_OK;

  BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.tq = tq; a.tk = tk; a.tv = tv; a.mask = mask; a.tmask = tmask;
  a.o = o; a.to = to; a.go = go; a.gto = gto; a.lse = lse; a.tlse = tlse;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dtq = dtq; a.dtk = dtk; a.dtv = dtv;
  a.ws = static_cast<float*>(workspace);
  a.ws_stride = bwd_workspace_bytes(sz.rows_q) / 16;   // bytes of one array / 4
  a.H = p->H; a.Nq = p->Nq; a.Nk = p->Nk; a.BH = p->B * p->H;
  a.grp = sz.group;
  a.BHK = p->B * sz.hkv;
  a.n_blk = 0;
  a.n_items = 0;
  a.max_wgs = walk_workgroups();
  a.dq_two = 0;
  a.msb = p->mask_stride_b; a.msh = p->mask_stride_h; a.msq = p->mask_stride_q;
  a.scale = p->scale;
  a.inv_scale = 1.0f / p->scale;
  a.mask_vec = 0;
  {
    const int mes = p->mask_kind == JVPATTN_MASK_BOOL ? 1 : elem_bytes(p->dtype);
    const uintptr_t base = reinterpret_cast<uintptr_t>(mask);
    const uintptr_t tbase = reinterpret_cast<uintptr_t>(tmask);   // read with the same offsets
    a.mask_vec = mask && (p->mask_stride_b % 4 == 0) && (p->mask_stride_h % 4 == 0) &&
                 (p->mask_stride_q % 4 == 0) && (base % (4 * mes) == 0) && (tbase % (4 * mes) == 0);
  }
  const bool additive = p->mask_kind == JVPATTN_MASK_ADDITIVE;
  int sexp = 0;
  const bool pow2 = p->dtype == JVPATTN_BF16 && std::frexp(p->scale, &sexp) == 0.5f;
  a.cx = (additive || pow2) ? kLog2e : p->scale * kLog2e;
  hipStream_t s = static_cast<hipStream_t>(stream);

  const int kind = tmask ? kMaskAddT : p->mask_kind;
  const jvpattn_dtype dt = static_cast<jvpattn_dtype>(p->dtype);
  const bool c = p->causal != 0;
  auto part = [&](auto which, hipStream_t st) {
    constexpr int W = decltype(which)::value;
    return p->d == 64 ? bwd_launch_part<W, 64>(a, sz.rows_q, dt, kind, c, pow2, st)
                      : bwd_launch_part<W, 128>(a, sz.rows_q, dt, kind, c, pow2, st);
  };
  using Rows = std::integral_constant<int, kLaunchRows>;
  using Dkv = std::integral_constant<int, kLaunchDkv>;
  using Dq = std::integral_constant<int, kLaunchDq>;
  const int mode = g_overlap.load(std::memory_order_relaxed);
  bool fork = may_fork && sz.rows_q > 0 && sz.rows_k > 0 && mode != 0;
  if (fork && mode < 0) {
    const int64_t items = (int64_t(p->Nk) + kBBlk - 1) / kBBlk * a.BHK;
    const int64_t cus = cu_count();
    fork = p->d == 128 || items < cus || (c && items < 2 * cus);
  }
  if (fork) {   // never inside a graph capture of the caller's stream
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t ce = hipStreamIsCapturing(s, &cs);
    if (ce != hipSuccess) {
      g_last_hip_error = static_cast<int>(ce);
      return JVPATTN_ERR_HIP;
    }
    fork = cs == hipStreamCaptureStatusNone;
  }
  // The query side at d = 64 on its two-workgroups-per-CU kernel once its grid
  // is four or more workgroups per CU and it has the chip to itself; the
  // pipelined kernel (one per CU) is faster on smaller grids and beside the
  // key side.
  {
    const int64_t qblocks = (int64_t(p->Nq) + kBBlk - 1) / kBBlk * a.BH;
    const int64_t cus = cu_count();
    a.dq_two = p->d == 64 && p->dtype != JVPATTN_F32 && !fork && cus > 0 && qblocks >= 4 * cus;
  }
  hipError_t e = part(Rows{}, s);
  if (e == hipSuccess && fork) {
    hipDevice_t dev = 0;
    e = hipStreamGetDevice(s, &dev);
    std::lock_guard<std::mutex> lock(g_side_mu);
    SideStream* x = nullptr;
    if (e == hipSuccess) e = side_stream(static_cast<int>(dev), &x);
    if (e == hipSuccess) e = hipEventRecord(x->rows, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(x->s, x->rows, 0);
    if (e == hipSuccess) e = part(Dkv{}, s);    // the key side is queued first
    if (e == hipSuccess) e = part(Dq{}, x->s);
    if (e == hipSuccess) e = hipEventRecord(x->done, x->s);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, x->done, 0);
  } else if (e == hipSuccess) {
    e = part(Dkv{}, s);
    if (e == hipSuccess) e = part(Dq{}, s);
  }
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return JVPATTN_ERR_HIP;
  }
  return JVPATTN_OK;
}

}  // namespace
}  // namespace jvpattn

extern "C" int jvpattn_bwd(const jvpattn_params* p, const void* q, const void* k, const void* v,
                           const void* tq, const void* tk, const void* tv, const void* mask, const void* o,
                           const void* to, const float* lse, const float* tlse, const void* go,
                           const void* gto, void* dq, void* dk, void* dv, void* dtq, void* dtk, void* dtv,
                           void* workspace, size_t workspace_bytes, void* stream) {
  using namespace jvpattn;
  FwdSizes sz;
  const int rc = check_bwd(p, q, k, v, tq, tk, tv, mask, o, to, lse, tlse, go, gto, dq, dk, dv, dtq, dtk, dtv,
                           workspace, workspace_bytes, &sz);
  if (rc != JVPATTN_OK) return rc;
  return bwd_launch(p, sz, q, k, v, tq, tk, tv, mask, nullptr, o, to, lse, tlse, go, gto, dq, dk, dv, dtq, dtk,
                    dtv, workspace, stream, true);
}

extern "C" int jvpattn_bwd_tmask(const jvpattn_params* p, const void* q, const void* k, const void* v,
                                 const void* tq, const void* tk, const void* tv, const void* mask,
                                 const void* tmask, const void* o, const void* to, const float* lse,
                                 const float* tlse, const void* go, const void* gto, void* dq, void* dk, void* dv,
                                 void* dtq, void* dtk, void* dtv, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  using namespace jvpattn;
  FwdSizes sz;
  const int rc = check_bwd_tmask(p, q, k, v, tq, tk, tv, mask, tmask, o, to, lse, tlse, go, gto, dq, dk, dv, dtq,
                                 dtk, dtv, workspace, workspace_bytes, &sz);
  if (rc != JVPATTN_OK) return rc;
  return bwd_launch(p, sz, q, k, v, tq, tk, tv, mask, tmask, o, to, lse, tlse, go, gto, dq, dk, dv, dtq, dtk,
                    dtv, workspace, stream, true);
}

// ------------------------------------------------- allocation-free variant
//
// jvpattn_bwd_noalloc keeps the four per-row arrays of the workspace in a
// file-scope device array instead of caller memory: each GPU the library runs
// on holds its own copy (16 MiB) until the process ends. Host code never uses
// the array's name as an address: the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
namespace jvpattn {
namespace {

constexpr int64_t kScratchRows = int64_t(1) << 20;                 // B * H * Nq at most
constexpr int64_t kScratchBytes = 4 * kScratchRows * 4;            // four float32 arrays of that many rows
static_assert(kScratchBytes % 256 == 0, "each array starts on a 256-byte boundary");

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace
}  // namespace jvpattn

static __device__ __align__(256) unsigned char scratch[jvpattn::kScratchBytes];

namespace jvpattn {
namespace {

// Device address of `scratch` on device `dev`, looked up on the first call for that device.
int scratch_of(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return JVPATTN_ERR_ARG;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* ptr = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess || !ptr) {
      g_last_hip_error = static_cast<int>(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return JVPATTN_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return JVPATTN_OK;
}

}  // namespace
}  // namespace jvpattn

extern "C" int jvpattn_bwd_noalloc(const jvpattn_params* p, const void* q, const void* k, const void* v,
                                   const void* tq, const void* tk, const void* tv, const void* mask, const void* o,
                                   const void* to, const float* lse, const float* tlse, const void* go,
                                   const void* gto, void* dq, void* dk, void* dv, void* dtq, void* dtk, void* dtv,
                                   void* stream) {
  using namespace jvpattn;
  // The size limit first, before any runtime call.
  const int64_t need = jvpattn_bwd_workspace_bytes(p);
  if (need < 0) return static_cast<int>(need);
  if (need > kScratchBytes) return JVPATTN_ERR_SCRATCH;
  hipDevice_t dev = 0;
  const hipError_t e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev);
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return JVPATTN_ERR_HIP;
  }
  void* ws = nullptr;
  int rc = scratch_of(static_cast<int>(dev), &ws);
  if (rc != JVPATTN_OK) return rc;
  FwdSizes sz;
  rc = check_bwd(p, q, k, v, tq, tk, tv, mask, o, to, lse, tlse, go, gto, dq, dk, dv, dtq, dtk, dtv, ws,
                 static_cast<size_t>(kScratchBytes), &sz);
  if (rc != JVPATTN_OK) return rc;
  return bwd_launch(p, sz, q, k, v, tq, tk, tv, mask, nullptr, o, to, lse, tlse, go, gto, dq, dk, dv, dtq, dtk,
                    dtv, ws, stream, false);   // no stream or event is created here
}

extern "C" int jvpattn_bwd_set_overlap(int mode) {
  if (mode < -1 || mode > 1) return JVPATTN_ERR_ARG;
  jvpattn::g_overlap.store(mode, std::memory_order_relaxed);
  return JVPATTN_OK;
}
