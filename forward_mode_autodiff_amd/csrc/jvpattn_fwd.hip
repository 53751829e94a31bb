// Forward entry points: validation (jvpattn_check.cpp), then the launch plan
// -- kernel family, grid order, key range -- and the typed launch, whose
// kernel instances live in jvpattn_fwd_inst.hip. What each kernel computes is
// described in jvpattn_fwd_kernels.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>

#include "jvpattn.h"
#include "jvpattn_fwd_launch.h"
#include "jvpattn_internal.h"

namespace jvpattn {
namespace {

constexpr int kBM = 128;      // query rows per 4-wave workgroup
constexpr int kPPBM = 256;    // query rows per ping-pong workgroup
constexpr float kLog2e = 1.4426950408889634f;

// Process-wide algorithm selection (jvpattn_fwd_set_algo); -1 = automatic.
std::atomic<int> g_algo_kernel{-1}, g_algo_order{-1}, g_algo_key_range{-1}, g_max_workgroups{0};

// Queue the forward for arguments already validated (sizes from the check).
// tmask: the additive mask's tangent, or NULL.
int fwd_launch(const jvpattn_params* p, const FwdSizes& sz, const void* q, const void* k, const void* v,
               const void* tq, const void* tk, const void* tv, const void* mask, const void* tmask, void* o,
               void* to, float* lse, float* tlse, void* stream) {
  if (sz.rows_q == 0) return JVPATTN_OK;

  FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.tq = tq; a.tk = tk; a.tv = tv; a.mask = mask; a.tmask = tmask;
  a.o = o; a.to = to; a.lse = lse; a.tlse = tlse;
  a.H = p->H; a.Nq = p->Nq; a.Nk = p->Nk; a.BH = p->B * p->H;
  // Head dimensions run on kernels built for 64, 128 or 256 columns; d = 32
  // and 96 run zero-padded to the next one (the padding reads as zeros, is
  // never stored, and adds nothing to any product).
  const int dphys = p->d <= 64 ? 64 : p->d <= 128 ? 128 : 256;
  a.dh = p->d;
  a.grow = p->d * elem_bytes(p->dtype);
  a.grp = sz.group;
  a.xgrp = (sz.group > 1 && a.BH % (8 * sz.group) == 0) ? sz.group : 1;
  a.n_qblk = (p->Nq + kBM - 1) / kBM;
  a.msb = p->mask_stride_b; a.msh = p->mask_stride_h; a.msq = p->mask_stride_q;
  a.scale = p->scale;
  a.inv_scale = 1.0f / p->scale;
  const bool additive = p->mask_kind == JVPATTN_MASK_ADDITIVE;
  // 16-bit types with a power-of-two scale: the scale is folded into Q and dQ
  // once (exact in bfloat16, which has float32's exponent range; in float16
  // exact unless a product falls below 2^-14, where it rounds to the subnormal
  // grid), scores and score tangents arrive scaled.
  int sexp = 0;
  const bool pow2 = p->dtype != JVPATTN_F32 && std::frexp(p->scale, &sexp) == 0.5f;
  // Otherwise scores stay raw (q.k) without an additive mask, so scale folds into cx.
  a.cx = (additive || pow2) ? kLog2e : p->scale * kLog2e;
  const float tau = p->dtype == JVPATTN_BF16 ? kTauBF16 : p->dtype == JVPATTN_F16 ? kTauF16 : kTauF32;
  a.thr = tau / a.cx;
  {
    const int mes = p->mask_kind == JVPATTN_MASK_BOOL ? 1 : elem_bytes(p->dtype);
    const uintptr_t base = reinterpret_cast<uintptr_t>(mask);
    const int64_t need = 4;  // keys per vector read
    const uintptr_t tbase = reinterpret_cast<uintptr_t>(tmask);   // read with the same offsets
    a.mask_vec = mask && (p->mask_stride_b % need == 0) && (p->mask_stride_h % need == 0) &&
                 (p->mask_stride_q % need == 0) && (base % (need * mes) == 0) && (tbase % (need * mes) == 0);
  }
  // Kernel choice for 16-bit d = 64: the 8-wave ping-pong kernel (256 rows per
  // workgroup) when it still gives every CU a workgroup; else the 4-wave
  // kernel (128 rows), with the key range split between two groups of waves
  // when it would have fewer than two workgroups per CU, and on 64-row blocks
  // (two groups of two waves) when even 128-row blocks leave CUs without one
  // -- or, causal, fewer than two: there twice the blocks, heaviest first,
  // even out the triangle. Other types and d: the 4-wave kernel (float32: its
  // own). jvpattn_fwd_set_algo can force a family.
  const int64_t n64 = (p->Nq + 63) / 64, n128 = (p->Nq + kBM - 1) / kBM, n256 = (p->Nq + kPPBM - 1) / kPPBM;
  const bool d64_16 = dphys == 64 && p->dtype != JVPATTN_F32;
  bool pp = d64_16 && n256 * a.BH >= 256;
  const int64_t small = p->causal ? 512 : 256;
  int split = !d64_16 || pp ? 0 : n128 * a.BH < small ? 2 : n128 * a.BH < 512 ? 1 : 0;
  // A forced family applies where it exists (the ping-pong and split kernels: 16-bit, d = 64).
  switch (g_algo_kernel.load(std::memory_order_relaxed)) {
    case JVPATTN_FWD_PINGPONG: pp = d64_16, split = 0; break;
    case JVPATTN_FWD_WG4: pp = false, split = 0; break;
    case JVPATTN_FWD_SPLIT: pp = false, split = d64_16 ? 1 : 0; break;
    case JVPATTN_FWD_SPLIT64: pp = false, split = d64_16 ? 2 : 0; break;
    default: break;
  }
  // d = 256 runs its own kernel on 64-row blocks
  a.n_qblk = static_cast<int>(dphys == 256 ? n64 : pp ? n256 : split == 2 ? n64 : n128);
  const int64_t blocks = int64_t(a.n_qblk) * a.BH;
  if (blocks > INT32_MAX) return JVPATTN_ERR_SHAPE;
  // Head-major order once the grid is several times what the chip holds at
  // once (at most 2 workgroups per CU x 256 CUs), so a head's query blocks
  // would otherwise run far apart in time and each re-read its key/value
  // tiles from HBM. jvpattn_fwd_set_algo can force either order.
  a.head_major = a.n_qblk > 1 && a.BH % 8 == 0 && blocks >= 4 * 512;
  // A mask with row stride 0 is the same for every query row: scan it once per
  // workgroup and skip the key tiles it hides entirely. jvpattn_fwd_set_algo
  // can switch off both mask early-outs (then every block runs).
  const bool mask_skips = g_algo_key_range.load(std::memory_order_relaxed) != 0;
  a.key_range = mask != nullptr && p->mask_stride_q == 0 && mask_skips;
  // Any mask: a wave skips the softmax and value products of a 32 x 32 block
  // its mask hides entirely (decided from the mask values it loads anyway).
  a.skip_hidden = mask_skips ? 1 : 0;

  const int order = g_algo_order.load(std::memory_order_relaxed);
  if (order == 0) a.head_major = 0;
  if (order == 1) a.head_major = a.n_qblk > 1 && a.BH % 8 == 0;
  // A mask with one row per query, on the ping-pong kernel (large grids): each
  // workgroup finds the key tiles some of its rows can see, scanning from both
  // ends until it meets a visible key; its Q loads are in flight meanwhile.
  // The small-grid kernels skip only the blocks a mask hides from a whole
  // wave: there the scan, one memory round trip before each workgroup's first
  // tile, costs more than it saves on a dense mask.
  a.row_range = mask != nullptr && p->mask_stride_q != 0 && mask_skips && pp;
  hipStream_t s = static_cast<hipStream_t>(stream);

  const int kernel = pp ? kFwdPingPong : split == 2 ? kFwdSplit64 : split == 1 ? kFwdSplit : kFwdWG4;
  const bool c = p->causal != 0;
  int mk = p->mask_kind;
  if (mk == JVPATTN_MASK_ADDITIVE && tmask) mk = kMaskAddT;
  // The mask-free 4-wave kernel at 128 columns (bfloat16, d = 96 / 128, scale
  // not a power of two) walks its row blocks with at most as many workgroups
  // as the chip holds at once (one per CU), a multiple of 8 so each keeps its
  // XCD: a block's loads then overlap the previous block's epilogue and
  // stores. With one block per workgroup both latencies are exposed.
  a.n_items = static_cast<int>(blocks);
  int64_t wgs = blocks;
  if (kernel == kFwdWG4 && mk == JVPATTN_MASK_NONE && p->dtype == JVPATTN_BF16 && dphys == 128 && !pow2) {
    const int64_t cap = walk_workgroups();
    if (cap > 0 && cap < blocks) wgs = cap;
  }
  const dim3 grid(static_cast<unsigned>(wgs));
  hipError_t e;
  switch (mk) {
    case JVPATTN_MASK_NONE:
      e = c ? launch_fwd<JVPATTN_MASK_NONE, true>(kernel, p->dtype, dphys, pow2, a, grid, s)
            : launch_fwd<JVPATTN_MASK_NONE, false>(kernel, p->dtype, dphys, pow2, a, grid, s);
      break;
    case JVPATTN_MASK_BOOL:
      e = c ? launch_fwd<JVPATTN_MASK_BOOL, true>(kernel, p->dtype, dphys, pow2, a, grid, s)
            : launch_fwd<JVPATTN_MASK_BOOL, false>(kernel, p->dtype, dphys, pow2, a, grid, s);
      break;
    case JVPATTN_MASK_BITS:
      e = c ? launch_fwd<JVPATTN_MASK_BITS, true>(kernel, p->dtype, dphys, pow2, a, grid, s)
            : launch_fwd<JVPATTN_MASK_BITS, false>(kernel, p->dtype, dphys, pow2, a, grid, s);
      break;
    case JVPATTN_MASK_ADDITIVE:
      e = c ? launch_fwd<JVPATTN_MASK_ADDITIVE, true>(kernel, p->dtype, dphys, pow2, a, grid, s)
            : launch_fwd<JVPATTN_MASK_ADDITIVE, false>(kernel, p->dtype, dphys, pow2, a, grid, s);
      break;
    default:
      e = c ? launch_fwd<kMaskAddT, true>(kernel, p->dtype, dphys, pow2, a, grid, s)
            : launch_fwd<kMaskAddT, false>(kernel, p->dtype, dphys, pow2, a, grid, s);
      break;
  }
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return JVPATTN_ERR_HIP;
  }
  return JVPATTN_OK;
}

}  // namespace

int cu_count() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cus[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 0) n = 0;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

int walk_workgroups() {
  const int forced = g_max_workgroups.load(std::memory_order_relaxed);
  int cap = forced > 0 ? forced : cu_count();
  if (cap >= 8) cap &= ~7;
  return cap;
}

}  // namespace jvpattn

extern "C" int jvpattn_fwd(const jvpattn_params* p, const void* q, const void* k, const void* v,
                           const void* tq, const void* tk, const void* tv, const void* mask, void* o,
                           void* to, float* lse, float* tlse, void* stream) {
  using namespace jvpattn;
  FwdSizes sz;
  const int rc = check_fwd(p, q, k, v, tq, tk, tv, mask, o, to, lse, tlse, &sz);
  if (rc != JVPATTN_OK) return rc;
  return fwd_launch(p, sz, q, k, v, tq, tk, tv, mask, nullptr, o, to, lse, tlse, stream);
}

extern "C" int jvpattn_fwd_tmask(const jvpattn_params* p, const void* q, const void* k, const void* v,
                                 const void* tq, const void* tk, const void* tv, const void* mask,
                                 const void* tmask, void* o, void* to, float* lse, float* tlse, void* stream) {
  using namespace jvpattn;
  FwdSizes sz;
  const int rc = check_fwd_tmask(p, q, k, v, tq, tk, tv, mask, tmask, o, to, lse, tlse, &sz);
  if (rc != JVPATTN_OK) return rc;
  return fwd_launch(p, sz, q, k, v, tq, tk, tv, mask, tmask, o, to, lse, tlse, stream);
}

extern "C" int jvpattn_set_workgroups(int max_workgroups) {
  using namespace jvpattn;
  if (max_workgroups < 0) return JVPATTN_ERR_ARG;
  g_max_workgroups.store(max_workgroups, std::memory_order_relaxed);
  return JVPATTN_OK;
}

extern "C" int jvpattn_fwd_set_algo(int kernel, int order, int key_range) {
  using namespace jvpattn;
  if (kernel < -1 || kernel > JVPATTN_FWD_SPLIT64 || order < -1 || order > 1 || key_range < -1 || key_range > 1)
    return JVPATTN_ERR_ARG;
  g_algo_kernel.store(kernel, std::memory_order_relaxed);
  g_algo_order.store(order, std::memory_order_relaxed);
  g_algo_key_range.store(key_range, std::memory_order_relaxed);
  return JVPATTN_OK;
}
