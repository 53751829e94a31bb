// Fused attention forward with tangents for gfx950 (MI355X).
//
// One pass over the keys computes, per query row i,
//   O_i  = sum_j P_ij V_j,               P = softmax_j(scale q_i.k_j + M_ij)
//   dO_i = sum_j P_ij (dS_ij - tlse_i) V_j + sum_j P_ij dV_j
//   tlse_i = sum_j P_ij dS_ij,           dS_ij = scale (dq_i.k_j + q_i.dk_j)
// which is the Jacobian-vector product of scaled-dot-product attention (the
// "JVP Flash Attention" README, sections "Description" and "Usage").
//
// Streaming form (the N x N score matrix never exists in memory): keep per
// row a reference maximum m, l = sum e, mu = sum e dS, and two accumulators
// accO = sum e V and accT = sum e dS V + sum e dV, with e = exp(s - m).
// Then O = accO / l, tlse = mu / l, dO = accT / l - tlse O: dividing the
// streamed sums by l turns e into P, so this is the closed form above; a
// change of m multiplies every sum by the same factor and cancels.
//
// Mapping onto the matrix cores. Each wave owns 32 query rows and computes
// the transposed score block S^T = K Q^T (32 keys x 32 queries) with
// v_mfma_f32_32x32x16_{bf16,f16}. In the C layout of that instruction lane
// l holds column l%32 -- one query -- and 16 keys in its registers, so the
// row statistics need only in-lane reductions plus one exchange between
// lanes l and l^32, and the 16 registers, rounded to 16 bits, are already
// the B operand of the next product O^T += V^T P^T with no lane shuffles.
// V^T and dV^T A operands come from LDS transpose reads of the row-major
// key tiles.
// The score tangent uses one chain over 2d: dS^T = dK Q^T + K dQ^T.
// The two tangent products share one accumulator: accT += V^T (P dS)^T + dV^T P^T.
//
// This header holds the device code of every forward kernel and the typed
// launchers; jvpattn_fwd_inst.hip instantiates them once per (mask kind,
// causal) pair in separate objects, and jvpattn_fwd.hip plans the launch.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "jvpattn.h"
#include "jvpattn_device.h"
#include "jvpattn_fwd_launch.h"

namespace jvpattn {
namespace {


constexpr int kWaves = 4;             // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;      // query rows per workgroup

static_assert(kThreads == kTileThreads, "LDS tiles are laid out for the 4-wave kernels");


// Workgroup -> (query block, query head). Workgroups are dealt round-robin
// over the 8 XCDs, each with its own L2, so the mapping decides which blocks
// share cached key/value tiles.
//  - Default (the grid fits on the chip in a few rounds): query blocks run
//    heaviest first (causal work grows with the block index) and heads are
//    innermost; with B*H a multiple of 8 every block of a head lands on one
//    XCD, and all of them are resident together.
//  - head_major (grids many times the chip, B*H a multiple of 8): XCD x
//    runs heads x, x+8, ... one after the other, each head's query blocks
//    back to back (heaviest first), so they stream the same key/value tiles
//    at the same time and all but the first read them from L2 rather than
//    HBM.
// With grouped key/value heads (xgrp > 1, B*H a multiple of 8*xgrp) the heads
// are then permuted so that all query heads sharing a key/value head also
// land on one XCD.
__device__ inline void block_coords(const FwdArgs& a, int x, int& qb, int& bh) {
  int r;
  if (a.head_major) {
    const int slot = x >> 3;
    qb = a.n_qblk - 1 - slot % a.n_qblk;
    r = (slot / a.n_qblk) * 8 + (x & 7);
  } else {
    qb = a.n_qblk - 1 - x / a.BH;
    r = x % a.BH;
  }
  if (a.xgrp > 1) {
    const int xcd = r & 7, j = r >> 3;
    bh = ((j / a.xgrp) * 8 + xcd) * a.xgrp + j % a.xgrp;
  } else {
    bh = r;
  }
}

// Whether query row q (< Nq) of this head sees any key of 32-key tile t under
// a mask with one row per query (row stride msq). Keys past Nk do not count
// (their bytes belong to row padding or the next row).
template <typename T, int MASK, int ES>
__device__ inline bool row_tile_visible(const FwdArgs& a, Rsrc mr, int q, int t) {
  const int k0 = 32 * t;
  const int nk = min(32, a.Nk - k0);   // keys of this tile inside Nk (>= 1)
  if constexpr (MASK == JVPATTN_MASK_BITS) {
    uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(mr, (q * int(a.msq) + t) * 4, 0, 0);
    if (nk < 32) w &= (1u << nk) - 1u;
    return w != 0u;
  } else if constexpr (MASK == JVPATTN_MASK_BOOL) {
    const int base = q * int(a.msq) + k0;
    uint32_t any = 0u;
    if (a.mask_vec) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(mr, base + 4 * i, 0, 0);
        if (4 * i + 4 > nk) w = 4 * i >= nk ? 0u : w & ((1u << (8 * (nk - 4 * i))) - 1u);
        any |= w;
      }
    } else {
      for (int j = 0; j < nk; ++j) any |= __builtin_amdgcn_raw_buffer_load_b8(mr, base + j, 0, 0);
    }
    return any != 0u;
  } else {   // additive (and its tangent's kind): a key is hidden by -inf
    const int base = (q * int(a.msq) + k0) * ES;
    bool vis = false;
    if constexpr (ES == 2) {
      if (a.mask_vec) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(mr, base + 4 * i, 0, 0);
          vis = vis || (2 * i < nk && (w & 0xffffu) != T::kNegInf16) || (2 * i + 1 < nk && (w >> 16) != T::kNegInf16);
        }
      } else {
        for (int j = 0; j < nk; ++j)
          vis = vis || uint32_t(__builtin_amdgcn_raw_buffer_load_b16(mr, base + 2 * j, 0, 0)) != T::kNegInf16;
      }
    } else {
      for (int j = 0; j < nk; ++j)
        vis = vis || __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(mr, base + 4 * j, 0, 0)) != -INFINITY;
    }
    return vis;
  }
}

// The key tiles [t_lo, t_hi) within [0, tmax) that hold a key visible to some
// row q0 .. q0+nrows-1 (< Nq) under a mask with one row per query. The
// workgroup checks R tiles at a time from each end (both ends together in the
// first round) and stops at the first visible tile from the front and from
// the back, so the cost grows with the hidden tiles skipped, and a mask with
// visible keys near both ends (a dense random mask) costs one round. No
// visible key: t_lo = t_hi = 0. Every thread takes part; the result is uniform.
template <typename T, int MASK, int ES>
__device__ inline void row_tiles(const FwdArgs& a, Rsrc mr, int* red, int q0, int nrows, int tmax, int& t_lo,
                                 int& t_hi) {
  constexpr int R = MASK == JVPATTN_MASK_BITS ? 8 : MASK == JVPATTN_MASK_BOOL ? 4 : 2;   // tiles per round
  const int nthr = int(blockDim.x), tid = int(threadIdx.x);
  nrows = max(0, min(nrows, a.Nq - q0));
  const int pairs = R * nrows;   // (row, tile) checks per end per round
  int lo_base = 0, hi_top = tmax;
  t_lo = -1;
  t_hi = -1;
  while (t_lo < 0 || t_hi < 0) {
    if (tid == 0) {
      red[0] = INT32_MAX;
      red[1] = -1;
    }
    __syncthreads();
    int lo = INT32_MAX, hi = -1;
    for (int p = tid; p < pairs; p += nthr) {
      const int r = p % nrows, j = p / nrows;
      if (t_lo < 0) {
        const int t = lo_base + j;
        if (t < tmax && row_tile_visible<T, MASK, ES>(a, mr, q0 + r, t)) lo = min(lo, t);
      }
      if (t_hi < 0) {
        const int t = hi_top - 1 - j;
        if (t >= 0 && row_tile_visible<T, MASK, ES>(a, mr, q0 + r, t)) hi = max(hi, t);
      }
    }
    if (lo != INT32_MAX) atomicMin(&red[0], lo);
    if (hi >= 0) atomicMax(&red[1], hi);
    __syncthreads();
    const int glo = red[0], ghi = red[1];
    __syncthreads();
    if (t_lo < 0) {
      if (glo != INT32_MAX) t_lo = glo;
      lo_base += R;
      if (t_lo < 0 && lo_base >= tmax) t_lo = tmax;   // nothing visible from the front
    }
    if (t_hi < 0) {
      if (ghi >= 0) t_hi = ghi + 1;
      hi_top -= R;
      if (t_hi < 0 && hi_top <= 0) t_hi = 0;
    }
  }
  if (t_lo >= t_hi) t_lo = t_hi = 0;
}

// Tiles of 32 keys [t_lo, t_hi) that hold every key a row of this head may
// see. With a mask shared by all query rows (row stride 0: a key-padding mask
// [B,1,1,Nk] or [B,H,1,Nk]) the workgroup scans that one row and the loops
// start and end at the first and last tile with a visible key, so tiles the
// mask hides entirely are never loaded or multiplied (a row with no visible
// key at all gets no tile). With one mask row per query (row_range), the
// range of tiles visible to some row of this workgroup's rows q0 .. q0+nrows-1
// (row_tiles). Otherwise every tile: [0, ceil(Nk/32)). Every thread of the
// workgroup takes part; the result is uniform. ES: bytes per mask element
// (additive masks hide a key with -inf).
template <typename T, int MASK, int ES>
__device__ inline void key_tiles(const FwdArgs& a, Rsrc mr, int* red, int& t_lo, int& t_hi, int q0, int nrows,
                                 bool causal) {
  t_lo = 0;
  t_hi = (a.Nk + 31) >> 5;
  if constexpr (MASK != JVPATTN_MASK_NONE) {
    if (a.row_range) {   // one mask row per query: this workgroup's rows, tile by tile from both ends
      const int tmax = causal ? min(t_hi, (q0 + nrows + 31) >> 5) : t_hi;
      row_tiles<T, MASK, ES>(a, mr, red, q0, nrows, tmax, t_lo, t_hi);
      return;
    }
    if (!a.key_range) return;
    if (threadIdx.x == 0) {
      red[0] = INT32_MAX;
      red[1] = -1;
    }
    __syncthreads();
    int lo = INT32_MAX, hi = -1;
    if constexpr (MASK == JVPATTN_MASK_BITS) {
      const int nw = (a.Nk + 31) >> 5;
      for (int j = threadIdx.x; j < nw; j += blockDim.x) {
        uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(mr, 4 * j, 0, 0);
        if (j == nw - 1 && (a.Nk & 31)) w &= (1u << (a.Nk & 31)) - 1u;   // bits past Nk
        if (w) {
          lo = min(lo, 32 * j + int(__builtin_ctz(w)));
          hi = max(hi, 32 * j + 31 - int(__builtin_clz(w)));
        }
      }
    }
    for (int j = threadIdx.x; MASK != JVPATTN_MASK_BITS && j < a.Nk; j += blockDim.x) {
      bool vis;
      if constexpr (MASK == JVPATTN_MASK_BOOL || MASK == JVPATTN_MASK_BITS) {
        vis = __builtin_amdgcn_raw_buffer_load_b8(mr, j, 0, 0) != 0;
      } else if constexpr (ES == 2) {
        vis = T::widen(__builtin_amdgcn_raw_buffer_load_b16(mr, 2 * j, 0, 0)) != -INFINITY;
      } else {
        vis = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(mr, 4 * j, 0, 0)) != -INFINITY;
      }
      if (vis) {
        lo = min(lo, j);
        hi = max(hi, j);
      }
    }
    if (hi >= 0) {
      atomicMin(&red[0], lo);
      atomicMax(&red[1], hi);
    }
    __syncthreads();
    hi = red[1];
    t_lo = hi < 0 ? 0 : red[0] >> 5;
    t_hi = hi < 0 ? 0 : (hi >> 5) + 1;
  }
}


// Per-row softmax state for one lane (both lanes of a query column hold the same m).
struct RowState {
  float m;       // reference maximum in score units (-inf until a visible key is seen)
  float moff;    // m * cx, or 0 while m is -inf
  float l;       // partial sum of weights over this lane's keys
  float mu;      // partial sum of weights * score tangent (in the units of sd)
};


template <typename T, int MASK, bool CAUSAL, bool PRESCALED>
__device__ inline void mask_scores(f32x16& s, const FwdArgs& a, Rsrc mr, int qi, int k0, int hlf,
                                   bool elem_mask) {
  MaskVals<MASK> m;
  mask_load<MASK>(m, a, mr, qi, k0, hlf);
  mask_apply<T, MASK, PRESCALED>(s, m, a.scale);
  if (elem_mask) hide_keys<CAUSAL>(s, a.Nk, qi, k0, hlf);
}

// Move the reference maximum when some row of the wave saw a score more than
// thr above it. Returns alpha != 1 (and true) when accumulators must be scaled.
__device__ inline bool update_max(float bm, RowState& st, float cx, float thr, float& alpha) {
  alpha = 1.0f;
  const bool need = bm > st.m + thr;
  if (!__any(need)) return false;
  const float mn = fmaxf(st.m, bm);
  alpha = mn == -INFINITY ? 1.0f : exp2f((st.m - mn) * cx);
  st.l *= alpha;
  st.mu *= alpha;
  st.m = mn;
  st.moff = mn == -INFINITY ? 0.0f : mn * cx;
  return true;
}

// Weights e = exp(s - m) (into s) and e * sd (into sd); their sums into l, mu.
__device__ inline void exp_block(f32x16& s, f32x16& sd, RowState& st, float cx) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], cx, -st.moff));
    sd[r] *= s[r];
  }
  float l0 = s[0] + s[1], l1 = s[2] + s[3], m0 = sd[0] + sd[1], m1 = sd[2] + sd[3];
#pragma unroll
  for (int r = 4; r < 16; r += 4) {
    l0 += s[r] + s[r + 1];
    l1 += s[r + 2] + s[r + 3];
    m0 += sd[r] + sd[r + 1];
    m1 += sd[r + 2] + sd[r + 3];
  }
  st.l += l0 + l1;
  st.mu += m0 + m1;
}

// Weights e = exp(s - m) (into s); their lane sum is added to l and returned.
__device__ inline float exp_l(f32x16& s, RowState& st, float cx) {
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(fmaf(s[r], cx, -st.moff));
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = s[r];
  const float lt = sum16(x);
  st.l += lt;
  return lt;
}

// Online-softmax update for one 32-key block (float32 kernel).
__device__ inline bool softmax_block(f32x16& s, f32x16& sd, RowState& st, float cx, float thr,
                                     float& alpha) {
  const bool rescale = update_max(block_max(s), st, cx, thr, alpha);
  exp_block(s, sd, st, cx);
  return rescale;
}

// ------------------------------------------------------------- 16-bit kernel
//
// Software pipeline per wave over 32-key blocks k: while the vector units turn
// block k's scores into weights, the matrix cores already compute block k+1's
// scores; block k's value products follow. The reference maximum for block
// k+1 is settled at the end of iteration k, so the only branch in the steady
// state (a rare rescale) sits between iterations. Blocks that need per-key
// masking (the causal diagonal, a ragged tail) take a non-pipelined path.
//
// LDS holds a ring of 4 tiles, each fetched two iterations ahead; one
// workgroup barrier per tile. The four stages are separate arrays and the
// loop is unrolled by four, so every LDS access names its stage statically
// and in-flight loads into other stages never force a wait.

//
// SPLIT = 2 (small grids, d = 64): two groups of four waves per workgroup
// take the same 128 rows; group G streams the G-th half of the key blocks
// through its own ring, then group 1 hands its row state and accumulators to
// group 0 through LDS (x0..x3: group 1's stages, one 16 KB stage per wave;
// xst: m, moff, l, mu per lane), which combines the two online-softmax states -- rescaling
// each to the larger reference -- and stores. Twice the waves per row block.
//
// WV = waves per group (32 query rows each): 4, or 2 for grids too small to
// give every CU a 128-row block -- then 64-row blocks, twice the workgroups.
//
// `item` is the row block (through block_coords). A workgroup that walks
// several (the grid holds fewer workgroups than there are blocks) passes the
// next one as `next_item`: once its own loop is done it issues that block's
// Q / dQ loads (into qB / tqB, which the caller keeps) and first three tiles,
// then stores its results, so the next block's load latency overlaps this
// one's epilogue and stores; the next call then has `loaded` set.
// Whether the 4-wave kernel instance walks several row blocks per workgroup
// (bfloat16, mask-free, 128 columns, scale not folded into Q): elsewhere the
// extra state would spill registers (float16 keeps a guard of its own).
template <typename T, int D, int MASK, bool POW2, int SPLIT>
constexpr bool fwd16_walks() {
  return std::is_same_v<T, BF16> && SPLIT == 1 && MASK == JVPATTN_MASK_NONE && D == 128 && !POW2;
}
template <bool FIRST, typename X>
__device__ __forceinline__ X& pick(X& a, X& b) {
  if constexpr (FIRST) return a;
  else return b;
}

template <typename T, int D, int MASK, bool CAUSAL, bool POW2, int SPLIT, int G, int WV>
__device__ __forceinline__ void fwd16_body(const FwdArgs& a, int item, int next_item, bool loaded,
                                           typename T::vec8 (&qBw)[Tile16<D>::NC],
                                           typename T::vec8 (&tqBw)[Tile16<D>::NC], int t_lo, int t_hi,
                                           char* stage0, char* stage1, char* stage2, char* stage3, char* x0,
                                           char* x1, char* x2, char* x3, float4* xst) {
  using L = Tile16<D>;
  using vec8 = typename T::vec8;
  // Q / dQ registers: the caller's when the workgroup walks blocks (they carry
  // the next block's values over), else the body's own (the compiler keeps
  // those in registers more tightly).
  constexpr bool WALK = fwd16_walks<T, D, MASK, POW2, SPLIT>();
  // A walking block's epilogue stores, the same count in every wave: O and
  // dO per 4 x 4 tile group, lse, tlse.
  constexpr int kEpStores = 2 * 4 * L::NT + 2;
  // Direct loads that bring a walking block's 32 Q (and dQ) rows of this wave into LDS.
  constexpr int kQDma = 32 * L::ROW / 1024;
  vec8 qBl[L::NC], tqBl[L::NC];
  vec8(&qB)[L::NC] = pick<WALK>(qBw, qBl);
  vec8(&tqB)[L::NC] = pick<WALK>(tqBw, tqBl);
  constexpr int GT = 64 * WV;                           // threads per group
  constexpr int BMG = 32 * WV;                          // query rows per workgroup
  constexpr int LOADS = L::TENSOR_BYTES / (16 * GT);    // 16-byte tile loads per thread per tensor
  constexpr int TILE_VMEM = 4 * LOADS;                  // direct loads per thread per tile
  static_assert(LOADS * 16 * GT == L::TENSOR_BYTES, "tile must split evenly over the group");

  const int tid = threadIdx.x & (GT - 1);   // thread within the group
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave within the group
  const int c32 = lane & 31;
  const int hlf = lane >> 5;

  int qb, bh;
  block_coords(a, item, qb, bh);
  const int b = bh / a.H, h = bh % a.H;
  const int q0 = qb * BMG;
  const int qw0 = q0 + 32 * wave;
  const int qi = qw0 + c32;
  const bool wave_live = qw0 < a.Nq;

  // Global rows hold a.dh <= D logical columns (a.grow bytes); the kernel works on D columns, the
  // ones past a.dh read as zeros (an out-of-range buffer offset) and are never stored.
  const int64_t qhead = int64_t(bh) * a.Nq * a.grow;   // byte offsets of this head
  const int64_t khead = int64_t(bh / a.grp) * a.Nk * a.grow;   // the key/value head it reads
  const char* qp = static_cast<const char*>(a.q) + qhead;
  const char* kp = static_cast<const char*>(a.k) + khead;
  const char* vp = static_cast<const char*>(a.v) + khead;
  const char* tqp = a.tq ? static_cast<const char*>(a.tq) + qhead : qp;
  const char* tkp = a.tk ? static_cast<const char*>(a.tk) + khead : kp;
  const char* tvp = a.tv ? static_cast<const char*>(a.tv) + khead : vp;
  const int64_t qbytes = int64_t(a.Nq) * a.grow;

  // Q and dQ as B operands: lane holds row qi, head-dim entries hlf*D/2 + 8c .. +7.
  // With POW2 the scale (a power of two) is folded into them (T::scale8); a
  // workgroup that walks several blocks (never with POW2) loads them ahead.
  auto load_q = [&](const char* qp_, const char* tqp_, int qi_) {
    const Rsrc rq = make_rsrc(qp_, qbytes), rtq = make_rsrc(tqp_, a.tq ? qbytes : 0);
#pragma unroll
    for (int c = 0; c < L::NC; ++c) {
      const int col = hlf * (D / 2) + 8 * c;
      const int off = col < a.dh ? qi_ * a.grow + col * 2 : kOutOfRange;
      qB[c] = __builtin_bit_cast(vec8, ld128(rq, off));
      tqB[c] = __builtin_bit_cast(vec8, ld128(rtq, off));
      if constexpr (POW2) {
        qB[c] = T::scale8(qB[c], a.scale);
        tqB[c] = T::scale8(tqB[c], a.scale);
      }
    }
  };
  if (!loaded) load_q(qp, tqp, qi);

  f32x16 accO[L::NT], accT[L::NT];
#pragma unroll
  for (int t = 0; t < L::NT; ++t) {
    accO[t] = f32x16{};
    accT[t] = f32x16{};
  }
  RowState st{-INFINITY, 0.0f, 0.0f, 0.0f};
  const Rsrc mr = mask_rsrc(a, b, h, mask_es<MASK>(2), nullptr, MASK == JVPATTN_MASK_BITS);
  const Rsrc mtr = MASK == kMaskAddT ? mask_rsrc(a, b, h, 2, a.tmask) : mr;
  auto load_mask = [&](MaskVals<MASK>& m, int k0) {
    if constexpr (MASK == kMaskAddT) mask_load_t(m, a, mr, mtr, qi, k0, hlf);
    else mask_load<MASK>(m, a, mr, qi, k0, hlf);
  };
  const float inv_us = POW2 ? 1.0f : a.inv_scale;   // mask tangent -> units of sd

  const int kv_end = min(CAUSAL ? min(a.Nk, q0 + BMG) : a.Nk, 32 * t_hi);
  const int n_all = max(0, (kv_end + L::BN - 1) / L::BN - t_lo);
  // This group's key blocks kb .. kb+n_tiles-1 (absolute); both groups run
  // n_loop iterations (one barrier each), the shorter one idling through the
  // extra ones.
  const int n_first = SPLIT == 2 ? (n_all + 1) / 2 : n_all;
  const int kb = t_lo + (G == 1 ? n_first : 0);
  const int n_tiles = G == 1 ? n_all - n_first : n_first;
  const int n_loop = n_first;
  // Last block this wave needs (the causal diagonal block, or the last tile), absolute, then
  // local to this group; -1 if none.
  const int last_all = !wave_live ? -1 : (CAUSAL ? min(t_lo + n_all - 1, qw0 >> 5) : t_lo + n_all - 1);
  const int last = last_all < kb ? -1 : min(last_all - kb, n_tiles - 1);
  auto needs_keymask = [&](int k) {
    return (CAUSAL && (kb + k) * 32 + 31 > qw0) || ((kb + k) * 32 + 32 > a.Nk);
  };

  // Direct-load slots of this thread: global byte offset inside a 32-key tile (same for all four
  // tensors; kOutOfRange for granules past the logical columns), slot p of the LDS tile.
  int dl_off[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int p = i * GT + tid;
    const int row = p / L::GR, pg = p % L::GR, lg = pg ^ swz(row);
    dl_off[i] = lg < (a.dh >> 3) ? row * a.grow + (lg << 4) : kOutOfRange;
  }
  const int tile_g = L::BN * a.grow;   // global bytes of one 32-key tile
  // One buffer resource per tensor for the whole head: offsets past Nk rows
  // (ragged tail) or into an absent tangent (0-byte resource) read as zeros.
  const int64_t kbytes = int64_t(a.Nk) * a.grow;
  struct KvRsrc {
    Rsrc k, tk, v, tv;
  };
  auto kv_rsrc = [&](const char* kp_, const char* tkp_, const char* vp_, const char* tvp_) {
    return KvRsrc{make_rsrc(kp_, kbytes), make_rsrc(tkp_, a.tk ? kbytes : 0), make_rsrc(vp_, kbytes),
                  make_rsrc(tvp_, a.tv ? kbytes : 0)};
  };
  const KvRsrc kv = kv_rsrc(kp, tkp, vp, tvp);
  auto issue_from = [&](const KvRsrc& r, int kb_, int j, char* stage) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int off = dl_off[i] == kOutOfRange ? kOutOfRange : (kb_ + j) * tile_g + dl_off[i];
      const int slot = (i * GT + wave * 64) * 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r.k, (__attribute__((address_space(3))) void*)to_lds(stage + slot),
                                               16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r.tk, (__attribute__((address_space(3))) void*)to_lds(stage + L::TENSOR_BYTES + slot), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r.v, (__attribute__((address_space(3))) void*)to_lds(stage + 2 * L::TENSOR_BYTES + slot), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r.tv, (__attribute__((address_space(3))) void*)to_lds(stage + 3 * L::TENSOR_BYTES + slot), 16, off, 0, 0, 0);
    }
  };
  auto issue_tile = [&](int j, char* stage) { issue_from(kv, kb, j, stage); };

  // LDS read offsets of this lane (constant over the loop).
  // K / dK A operand, chunk c: row c32, logical granule hlf*NC + c.
  int kofs[L::NC];
#pragma unroll
  for (int c = 0; c < L::NC; ++c) kofs[c] = c32 * L::ROW + (((hlf * L::NC + c) ^ swz(c32)) << 4);
  // V^T / dV^T A operand via transpose reads: lane (group g16 = lane/16, i = lane%16) addresses
  // row 4*hlf + i/4 (+16 kc; vofs1 is the second read, 8 rows further), columns 32t + 16(g16&1) + 4(i&3).
  // swz() depends on row bits 0..3 only, so +16 kc keeps the swizzle.
  int vofs0[L::NT], vofs1[L::NT];
  {
    const int g16 = lane >> 4, i16 = lane & 15;
    const int r0 = 4 * hlf + (i16 >> 2), r1 = r0 + 8;
#pragma unroll
    for (int t = 0; t < L::NT; ++t) {
      const int gcol = 4 * t + 2 * (g16 & 1) + ((i16 & 3) >> 1);
      vofs0[t] = r0 * L::ROW + ((gcol ^ swz(r0)) << 4) + 8 * (i16 & 1);
      vofs1[t] = r1 * L::ROW + ((gcol ^ swz(r1)) << 4) + 8 * (i16 & 1);
    }
  }

  // K / dK operands of the tile at `sb`, and the score products S^T, dS^T.
  auto read_k = [&](const char* sb, vec8 (&ka)[L::NC], vec8 (&tka)[L::NC]) {
#pragma unroll
    for (int c = 0; c < L::NC; ++c) {
      ka[c] = __builtin_bit_cast(vec8, lds_load<uint4>(sb, kofs[c]));
      tka[c] = __builtin_bit_cast(vec8, lds_load<uint4>(sb + L::TENSOR_BYTES, kofs[c]));
    }
  };
  auto mma_s = [&](const vec8 (&ka)[L::NC], const vec8 (&tka)[L::NC], f32x16& s, f32x16& sd) {
    s = f32x16{};
    sd = f32x16{};
#pragma unroll
    for (int c = 0; c < L::NC; ++c) {
      s = T::mfma(ka[c], qB[c], s);
      sd = T::mfma(tka[c], qB[c], sd);
      sd = T::mfma(ka[c], tqB[c], sd);
    }
  };
  auto scores = [&](const char* sb, f32x16& s, f32x16& sd) {
    vec8 ka[L::NC], tka[L::NC];
    read_k(sb, ka, tka);
    mma_s(ka, tka, s, sd);
  };
  // At d = 128 the scaling goes tile by tile, each under its own opaque copy
  // of the flag: scaled in one block, all 128 accumulator registers would be
  // copied out of the AGPRs at once and the kernel would spill.
  auto rescale_acc = [&](bool rs, float alpha) {   // rs: uniform over the wave; alpha: per lane
#pragma unroll
    for (int t = 0; t < L::NT; ++t) {
      int rst = __builtin_amdgcn_readfirstlane(static_cast<int>(rs));
      if constexpr (D > 64) asm volatile("" : "+s"(rst));
      if (rst) {
        accO[t] *= alpha;
        accT[t] *= alpha;
      }
    }
  };
  auto rescale = [&](float bm) {
    float alpha;
    const bool rs = update_max(bm, st, a.cx, a.thr, alpha);
    if constexpr (D > 64) rescale_acc(rs, alpha);
    else if (rs) rescale_acc(true, alpha);
  };
  // Block weights: s -> e = exp(s - m), sd -> e * dS, packed as 16-bit B operands
  // for keys 16kc .. 16kc+15; l and mu updated.
  auto weights = [&](f32x16& s, f32x16& sd, vec8 (&pB)[2], vec8 (&uB)[2]) {
    const float lsum = exp_l(s, st, a.cx);
    if constexpr (__is_same(T, F16)) {
      const float moff0 = st.moff;
      const float shrink = f16_range_guard(s, sd, POW2 ? 1.0f : a.scale, lsum, st.moff, st.l, st.mu);
      if (shrink != 1.0f) st.m += (st.moff - moff0) / a.cx;
      if constexpr (D > 64) rescale_acc(__any(shrink != 1.0f), shrink);   // shrink is 1 on the other lanes
      else if (shrink != 1.0f) rescale_acc(true, shrink);
    }
    // the products e dS in float32: mu sums them, then they are rounded for the value products
    float u[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) u[r] = POW2 ? sd[r] * s[r] : (sd[r] * a.scale) * s[r];
    st.mu += sum16(u);
    uint32_t pw[8], uw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pw[i] = T::pack2(s[2 * i], s[2 * i + 1]);
      uw[i] = T::pack2(u[2 * i], u[2 * i + 1]);
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      pB[kc] = __builtin_bit_cast(vec8, uint4{pw[4 * kc], pw[4 * kc + 1], pw[4 * kc + 2], pw[4 * kc + 3]});
      uB[kc] = __builtin_bit_cast(vec8, uint4{uw[4 * kc], uw[4 * kc + 1], uw[4 * kc + 2], uw[4 * kc + 3]});
    }
  };
  // V^T / dV^T operands of the tile at `sb` (transpose reads) and the value
  // products accO += V^T P^T, accT += V^T U^T + dV^T P^T.
  auto read_v = [&](const char* sb, vec8 (&va)[L::NT][2], vec8 (&tva)[L::NT][2]) {
    const char* sv = sb + 2 * L::TENSOR_BYTES;
    const char* stv = sb + 3 * L::TENSOR_BYTES;
#pragma unroll
    for (int t = 0; t < L::NT; ++t)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const int o0 = 16 * kc * L::ROW + vofs0[t], o1 = 16 * kc * L::ROW + vofs1[t];
        va[t][kc] = __builtin_bit_cast(
            vec8, __builtin_shufflevector(lds_read_tr(sv + o0), lds_read_tr(sv + o1), 0, 1, 2, 3, 4, 5, 6, 7));
        tva[t][kc] = __builtin_bit_cast(
            vec8, __builtin_shufflevector(lds_read_tr(stv + o0), lds_read_tr(stv + o1), 0, 1, 2, 3, 4, 5, 6, 7));
      }
  };
  auto mma_v = [&](const vec8 (&va)[L::NT][2], const vec8 (&tva)[L::NT][2], const vec8 (&pB)[2],
                   const vec8 (&uB)[2]) {
#pragma unroll
    for (int t = 0; t < L::NT; ++t)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        accO[t] = T::mfma(va[t][kc], pB[kc], accO[t]);
        accT[t] = T::mfma(va[t][kc], uB[kc], accT[t]);
        accT[t] = T::mfma(tva[t][kc], pB[kc], accT[t]);
      }
  };
  auto values = [&](const char* sb, const vec8 (&pB)[2], const vec8 (&uB)[2]) {
    vec8 va[L::NT][2], tva[L::NT][2];
    read_v(sb, va, tva);
    mma_v(va, tva, pB, uB);
  };

  // Blocks 1.. that need per-key masking start at jm: the causal diagonal, a
  // ragged last tile, or the end of this wave's range.
  int jm = last + 1;
  if (CAUSAL) jm = min(jm, (qw0 >> 5) - kb);
  jm = min(jm, (a.Nk >> 5) - kb);
  jm = max(jm, 1);

  bool hidden = false;   // the mask hides the current block from all of this wave's rows
  // Pipelined iteration k (block k settled in sc; block k+1 needs no key mask).
  auto fast = [&](int k, const char* cur, const char* nxt, char* dma, f32x16& sc, f32x16& sdc, f32x16& sn,
                  f32x16& sdn) {
    // Tile k+1 was fetched two iterations ago; tile k+2 may still be in flight.
    if (k + 2 < n_tiles) wait_vmcnt<TILE_VMEM>();
    else wait_vmcnt<0>();
    ring_barrier();   // tile k+1 visible to all; every wave is done with tile k-1 (the `dma` stage)
    MaskVals<MASK> mk1;
    load_mask(mk1, (kb + k + 1) * 32);   // before the fetch: keeps its wait short
    if (k + 3 < n_tiles) issue_tile(k + 3, dma);
    // All LDS operands first (their latency hides behind the first weights),
    // then the score products of block k+1 interleaved with block k's softmax
    // on the vector units, then block k's value products.
    vec8 ka[L::NC], tka[L::NC], va[L::NT][2], tva[L::NT][2], pB[2], uB[2];
    read_k(nxt, ka, tka);
    read_v(cur, va, tva);
    mma_s(ka, tka, sn, sdn);
    // a block the mask hides from all of this wave's rows needs no softmax: its weights are zeros
    if (MASK != JVPATTN_MASK_NONE && hidden) {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        pB[kc] = vec8{};
        uB[kc] = vec8{};
      }
    } else {
      weights(sc, sdc, pB, uB);
    }
    mma_v(va, tva, pB, uB);
    if constexpr (MASK != JVPATTN_MASK_NONE) hidden = a.skip_hidden && !__any(mask_any_visible<T, MASK>(mk1));
    mask_apply<T, MASK, POW2>(sn, mk1, a.scale);
    mask_tangent<T, MASK>(sdn, mk1, inv_us);
    const float bm = block_max(sn);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * L::NC, 0);           // K / dK reads
    __builtin_amdgcn_sched_group_barrier(0x100, 8 * L::NT, 0);           // V / dV transpose reads
    __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);                  // first weights
#pragma unroll
    for (int i = 0; i < 3 * L::NC; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // score product
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);                 // weights
    }
#pragma unroll
    for (int i = 0; i < 6 * L::NT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // value product
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);                 // max of block k+1
    }
    rescale(bm);
  };

  f32x16 sA, sdA, sB, sdB;
  // Prologue: tiles 0..2 in flight, wait for tile 0, settle block 0 if it needs no key mask.
  if (!loaded) {
    if (n_tiles > 0) issue_tile(0, stage0);
    if (n_tiles > 1) issue_tile(1, stage1);
    if (n_tiles > 2) issue_tile(2, stage2);
    if (n_tiles > 2) wait_vmcnt<2 * TILE_VMEM>();
    else if (n_tiles > 1) wait_vmcnt<TILE_VMEM>();
    else wait_vmcnt<0>();
  } else {
    // Q and dQ (in stages 2 and 3) and tiles 0, 1 came with the previous
    // block, ahead of its kEpStores stores, which may stay in flight. Each
    // wave reads its own rows; tile 2 goes into stage 2 once all have.
    if (n_tiles > 1) wait_vmcnt<TILE_VMEM + kEpStores>();
    else wait_vmcnt<kEpStores>();
    const int qo = wave * 32 * L::ROW + c32 * L::ROW + hlf * (L::ROW / 2);
#pragma unroll
    for (int c = 0; c < L::NC; ++c) {
      qB[c] = __builtin_bit_cast(vec8, lds_load<uint4>(stage2, qo + 16 * c));
      tqB[c] = __builtin_bit_cast(vec8, lds_load<uint4>(stage3, qo + 16 * c));
    }
    ring_barrier();
    if (n_tiles > 2) issue_tile(2, stage2);
  }
  ring_barrier();
  bool ready = false;   // sA holds the current block's settled scores
  if (0 <= last && !needs_keymask(0)) {
    scores(stage0, sA, sdA);
    MaskVals<MASK> mk;
    load_mask(mk, kb * 32);
    if constexpr (MASK != JVPATTN_MASK_NONE) hidden = a.skip_hidden && !__any(mask_any_visible<T, MASK>(mk));
    mask_apply<T, MASK, POW2>(sA, mk, a.scale);
    mask_tangent<T, MASK>(sdA, mk, inv_us);
    rescale(block_max(sA));
    ready = true;
  }
  const int kfast = ready ? jm - 1 : 0;   // iterations 0 .. kfast-1 are pipelined
  int k = 0;
  for (; k + 4 <= kfast; k += 4) {
    fast(k, stage0, stage1, stage3, sA, sdA, sB, sdB);
    fast(k + 1, stage1, stage2, stage0, sB, sdB, sA, sdA);
    fast(k + 2, stage2, stage3, stage1, sA, sdA, sB, sdB);
    fast(k + 3, stage3, stage0, stage2, sB, sdB, sA, sdA);
  }
  if (k < kfast) {
    fast(k, stage0, stage1, stage3, sA, sdA, sB, sdB);
    if (k + 1 < kfast) fast(k + 1, stage1, stage2, stage0, sB, sdB, sA, sdA);
    if (k + 2 < kfast) fast(k + 2, stage2, stage3, stage1, sA, sdA, sB, sdB);
  }
  if (kfast & 1) {   // block kfast's scores were left in sB
    sA = sB;
    sdA = sdB;
  }

  // Remaining iterations (diagonal, ragged tail, and barrier-only ones past this
  // wave's range), one score buffer, stage chosen at run time.
  auto stage_of = [&](int i) -> char* {
    i &= 3;
    return i == 0 ? stage0 : i == 1 ? stage1 : i == 2 ? stage2 : stage3;
  };
  for (k = kfast; k < n_loop; ++k) {
    if (k + 2 < n_tiles) wait_vmcnt<TILE_VMEM>();
    else wait_vmcnt<0>();
    ring_barrier();
    if (k + 3 < n_tiles) issue_tile(k + 3, stage_of(k + 3));
    if (k > last) continue;
    const char* cur = stage_of(k);
    if (!ready) {
      scores(cur, sA, sdA);
      MaskVals<MASK> mk;
      load_mask(mk, (kb + k) * 32);
      if constexpr (MASK != JVPATTN_MASK_NONE) hidden = a.skip_hidden && !__any(mask_any_visible<T, MASK>(mk));
      mask_apply<T, MASK, POW2>(sA, mk, a.scale);
      mask_tangent<T, MASK>(sdA, mk, inv_us);
      if (needs_keymask(k)) hide_keys<CAUSAL>(sA, a.Nk, qi, (kb + k) * 32, hlf);
      rescale(block_max(sA));
    }
    ready = false;   // the next block, if any, is settled at the top of the next iteration
    if (MASK != JVPATTN_MASK_NONE && hidden) continue;
    vec8 pB[2], uB[2];
    weights(sA, sdA, pB, uB);
    values(cur, pB, uB);   // the next block, if any, is settled at the top of the next iteration
  }

  if constexpr (SPLIT == 2) {
    // Group 1 hands over its state through its own stages, once every wave is
    // done reading them (first barrier); group 0 combines after the second.
    // Every tile load has completed: the last iterations wait for all of them.
    ring_barrier();
    float4* acc = reinterpret_cast<float4*>(wave == 0 ? x0 : wave == 1 ? x1 : wave == 2 ? x2 : x3);
    if constexpr (G == 1) {
#pragma unroll
      for (int t = 0; t < L::NT; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          acc[((2 * t) * 4 + g) * 64 + lane] = float4{accO[t][4 * g], accO[t][4 * g + 1], accO[t][4 * g + 2],
                                                      accO[t][4 * g + 3]};
          acc[((2 * t + 1) * 4 + g) * 64 + lane] = float4{accT[t][4 * g], accT[t][4 * g + 1],
                                                          accT[t][4 * g + 2], accT[t][4 * g + 3]};
        }
      xst[wave * 64 + lane] = float4{st.m, st.moff, st.l, st.mu};
      ring_barrier();
      return;
    } else {
      ring_barrier();
      const float4 o = xst[wave * 64 + lane];
      const float m = fmaxf(st.m, o.x);   // -inf only if neither half saw a visible key
      const float a0 = st.m == -INFINITY ? 0.0f : exp2f((st.m - m) * a.cx);
      const float a1 = o.x == -INFINITY ? 0.0f : exp2f((o.x - m) * a.cx);
#pragma unroll
      for (int t = 0; t < L::NT; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 xo = acc[((2 * t) * 4 + g) * 64 + lane];
          const float4 xt = acc[((2 * t + 1) * 4 + g) * 64 + lane];
          accO[t][4 * g] = accO[t][4 * g] * a0 + xo.x * a1;
          accO[t][4 * g + 1] = accO[t][4 * g + 1] * a0 + xo.y * a1;
          accO[t][4 * g + 2] = accO[t][4 * g + 2] * a0 + xo.z * a1;
          accO[t][4 * g + 3] = accO[t][4 * g + 3] * a0 + xo.w * a1;
          accT[t][4 * g] = accT[t][4 * g] * a0 + xt.x * a1;
          accT[t][4 * g + 1] = accT[t][4 * g + 1] * a0 + xt.y * a1;
          accT[t][4 * g + 2] = accT[t][4 * g + 2] * a0 + xt.z * a1;
          accT[t][4 * g + 3] = accT[t][4 * g + 3] * a0 + xt.w * a1;
        }
      st.l = st.l * a0 + o.z * a1;
      st.mu = st.mu * a0 + o.w * a1;
      st.m = m;
      st.moff = m == -INFINITY ? 0.0f : m * a.cx;
    }
  }

  if (WALK && next_item >= 0) {
    // The next block's Q, dQ and first tiles, once every wave is done with the ring.
    ring_barrier();
    int qb2, bh2;
    block_coords(a, next_item, qb2, bh2);
    const int64_t qh2 = int64_t(bh2) * a.Nq * a.grow, kh2 = int64_t(bh2 / a.grp) * a.Nk * a.grow;
    const char* qp2 = static_cast<const char*>(a.q) + qh2;
    const char* kp2 = static_cast<const char*>(a.k) + kh2;
    const char* vp2 = static_cast<const char*>(a.v) + kh2;
    // Q and dQ rows straight into LDS (stages 2 and 3, this wave's 32 rows
    // each; no register waits for them here), then tiles 0 and 1.
    const Rsrc rq2 = make_rsrc(qp2, qbytes);
    const Rsrc rtq2 = make_rsrc(a.tq ? static_cast<const char*>(a.tq) + qh2 : qp2, a.tq ? qbytes : 0);
#pragma unroll
    for (int j = 0; j < kQDma; ++j) {
      const int r = j * (1024 / L::ROW) + lane / (L::ROW / 16), g = lane % (L::ROW / 16);
      const int off = g < (a.dh >> 3) ? (qb2 * BMG + 32 * wave + r) * a.grow + 16 * g : kOutOfRange;
      const int slot = wave * 32 * L::ROW + j * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq2, (__attribute__((address_space(3))) void*)to_lds(stage2 + slot),
                                               16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rtq2, (__attribute__((address_space(3))) void*)to_lds(stage3 + slot),
                                               16, off, 0, 0, 0);
    }
    const KvRsrc kv2 = kv_rsrc(kp2, a.tk ? static_cast<const char*>(a.tk) + kh2 : kp2, vp2,
                               a.tv ? static_cast<const char*>(a.tv) + kh2 : vp2);
    const int kv_end2 = min(CAUSAL ? min(a.Nk, qb2 * BMG + BMG) : a.Nk, 32 * t_hi);
    const int n2 = max(0, (kv_end2 + L::BN - 1) / L::BN - t_lo);
    if (n2 > 0) issue_from(kv2, t_lo, 0, stage0);
    if (n2 > 1) issue_from(kv2, t_lo, 1, stage1);
  }

  // Epilogue: combine the two lane halves of each query column, normalise, store.
  const float l = xhalf_sum(st.l);
  const float mu = xhalf_sum(st.mu);
  if constexpr (WALK) {
    // Every wave issues kEpStores stores (rows past Nq, columns past dh and
    // the second lane half's statistics land out of range and are dropped).
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const float tl = mu * inv;
    const int64_t hb = int64_t(bh) * a.Nq;
    const Rsrc ro = make_rsrc(static_cast<char*>(a.o) + hb * a.grow, qbytes);
    const Rsrc rto = make_rsrc(static_cast<char*>(a.to) + hb * a.grow, qbytes);
    const Rsrc rl = make_rsrc(a.lse + hb, int64_t(a.Nq) * 4);
    const Rsrc rtl = make_rsrc(a.tlse ? a.tlse + hb : a.lse, a.tlse ? int64_t(a.Nq) * 4 : 0);
    const bool row = qi < a.Nq;
#pragma unroll
    for (int t = 0; t < L::NT; ++t) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float ov[4], dv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ov[e] = accO[t][4 * g + e] * inv;
          dv[e] = accT[t][4 * g + e] * inv - tl * ov[e];
        }
        const int dd = 32 * t + 8 * g + 4 * hlf;
        const int off = row && dd < a.dh ? qi * a.grow + dd * 2 : kOutOfRange;
        st64(ro, off, uint2{T::pack2(ov[0], ov[1]), T::pack2(ov[2], ov[3])});
        st64(rto, off, uint2{T::pack2(dv[0], dv[1]), T::pack2(dv[2], dv[3])});
      }
    }
    const int soff = row && hlf == 0 ? qi * 4 : kOutOfRange;
    st32(rl, soff, __float_as_uint(l > 0.0f ? (st.moff + log2f(l)) * kLn2 : -INFINITY));
    st32(rtl, soff, __float_as_uint(tl));
  } else if (qi < a.Nq) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const float tl = mu * inv;   // mu sums e dS (float32 products)
    uint16_t* op = static_cast<uint16_t*>(a.o) + (int64_t(bh) * a.Nq + qi) * a.dh;
    uint16_t* top = static_cast<uint16_t*>(a.to) + (int64_t(bh) * a.Nq + qi) * a.dh;
#pragma unroll
    for (int t = 0; t < L::NT; ++t) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float ov[4], dv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ov[e] = accO[t][4 * g + e] * inv;
          dv[e] = accT[t][4 * g + e] * inv - tl * ov[e];
        }
        const int dd = 32 * t + 8 * g + 4 * hlf;
        if (dd < a.dh) {
          *reinterpret_cast<uint2*>(op + dd) = uint2{T::pack2(ov[0], ov[1]), T::pack2(ov[2], ov[3])};
          *reinterpret_cast<uint2*>(top + dd) = uint2{T::pack2(dv[0], dv[1]), T::pack2(dv[2], dv[3])};
        }
      }
    }
    if (hlf == 0) {
      const int64_t ri = int64_t(bh) * a.Nq + qi;
      a.lse[ri] = l > 0.0f ? (st.moff + log2f(l)) * kLn2 : -INFINITY;
      if (a.tlse) a.tlse[ri] = tl;
    }
  }
}

// The kernel bodies use gfx950 builtins; the host pass only needs the launch stubs.
template <typename T, int D, int MASK, bool CAUSAL, bool POW2, int SPLIT, int WV>
__global__ __launch_bounds__(64 * WV * SPLIT, (D == 64 && WV == 4) ? 2 : 1) void fwd16_kernel(FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using L = Tile16<D>;
  __shared__ __attribute__((aligned(16))) char s0[L::STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) char s1[L::STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) char s2[L::STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) char s3[L::STAGE_BYTES];
  // the key tiles this head may see, found once by the whole workgroup
  __shared__ int kred[2];
  int t_lo, t_hi;
  {
    int qb, bh;
    block_coords(a, int(blockIdx.x), qb, bh);
    const Rsrc mr = mask_rsrc(a, bh / a.H, bh % a.H, mask_es<MASK>(2), nullptr, MASK == JVPATTN_MASK_BITS);
    key_tiles<T, MASK, 2>(a, mr, kred, t_lo, t_hi, qb * 32 * WV, 32 * WV, CAUSAL);
  }
  using vec8 = typename T::vec8;
  vec8 qB[L::NC], tqB[L::NC];
  // A walking instance takes row blocks blockIdx.x + r * gridDim.x (the grid
  // may be smaller than their count); on odd rounds the workgroups of each
  // XCD take theirs in reverse, so heavy and light causal blocks pair up.
  if constexpr (fwd16_walks<T, D, MASK, POW2, SPLIT>()) {
    const int gsz = int(gridDim.x), b = int(blockIdx.x);
    const int brev = (gsz & 7) == 0 ? (gsz / 8 - 1 - b / 8) * 8 + (b & 7) : b;
    int it = b;
    for (int r = 0; it < a.n_items; ++r) {
      const int nx = (r + 1) * gsz + ((r & 1) ? b : brev);
      fwd16_body<T, D, MASK, CAUSAL, POW2, 1, 0, WV>(a, it, nx < a.n_items ? nx : -1, r > 0, qB, tqB, t_lo, t_hi,
                                                     s0, s1, s2, s3, nullptr, nullptr, nullptr, nullptr, nullptr);
      it = nx;
    }
  } else if constexpr (SPLIT == 1) {
    fwd16_body<T, D, MASK, CAUSAL, POW2, 1, 0, WV>(a, int(blockIdx.x), -1, false, qB, tqB, t_lo, t_hi, s0, s1, s2,
                                                   s3, nullptr, nullptr, nullptr, nullptr, nullptr);
  } else {
    __shared__ __attribute__((aligned(16))) char s4[L::STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) char s5[L::STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) char s6[L::STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) char s7[L::STAGE_BYTES];
    __shared__ float4 xst[kThreads];
    if (__builtin_amdgcn_readfirstlane(threadIdx.x / (64 * WV)) == 0)
      fwd16_body<T, D, MASK, CAUSAL, POW2, 2, 0, WV>(a, int(blockIdx.x), -1, false, qB, tqB, t_lo, t_hi, s0, s1,
                                                     s2, s3, s4, s5, s6, s7, xst);
    else
      fwd16_body<T, D, MASK, CAUSAL, POW2, 2, 1, WV>(a, int(blockIdx.x), -1, false, qB, tqB, t_lo, t_hi, s4, s5,
                                                     s6, s7, s4, s5, s6, s7, xst);
  }
#endif
}

// ------------------------------------------------ 16-bit ping-pong kernel (d = 64)
//
// Eight waves, 256 query rows per workgroup. Waves w and w+4 share a SIMD and
// are held in opposite phases by workgroup barriers: while group A (waves
// 0-3) issues only matrix-core work -- block i's value products and block
// i+1's score products -- group B (waves 4-7) runs the vector work of the
// previous iteration (mask, row maximum, exponentials, weights) and reads the
// LDS operands for its next matrix phase; then the roles swap. The matrix
// cores of each SIMD are fed by one wave while the other keeps the vector
// units busy. Group B also issues the tile loads, during its matrix phases.
//
// Tiles of 32 keys live in a ring of 6 LDS stages (separate arrays; the loop
// is unrolled by 6 so every access names its stage statically). Tile j is
// loaded at iteration j-6 and first read at iteration j-2.

constexpr int kPPWaves = 8;
constexpr int kPPThreads = 64 * kPPWaves;
constexpr int kPPBM = 32 * kPPWaves;
constexpr int kPPStages = 6;

template <typename T, int MASK, bool CAUSAL, bool POW2>
__device__ __forceinline__ void fwd16pp_body(const FwdArgs& a) {
  constexpr int D = 64;
  using L = Tile16<D>;
  using vec8 = typename T::vec8;
  static_assert(L::TILE_VMEM == 4, "group B loads a 32-key tile with 4 loads per thread");
  __shared__ __attribute__((aligned(16))) char stage0[L::STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) char stage1[L::STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) char stage2[L::STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) char stage3[L::STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) char stage4[L::STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) char stage5[L::STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool grp_b = wave >= 4;
  const int c32 = lane & 31;
  const int hlf = lane >> 5;

  int qb, bh;
  block_coords(a, int(blockIdx.x), qb, bh);
  const int b = bh / a.H, h = bh % a.H;
  const int q0 = qb * kPPBM;
  const int qw0 = q0 + 32 * wave;
  const int qi = qw0 + c32;
  const bool wave_live = qw0 < a.Nq;

  const int64_t qhead = int64_t(bh) * a.Nq * a.grow;   // global rows: a.dh columns (see fwd16_body)
  const int64_t khead = int64_t(bh / a.grp) * a.Nk * a.grow;   // the key/value head it reads
  const char* qp = static_cast<const char*>(a.q) + qhead;
  const char* kp = static_cast<const char*>(a.k) + khead;
  const char* vp = static_cast<const char*>(a.v) + khead;
  const char* tqp = a.tq ? static_cast<const char*>(a.tq) + qhead : qp;
  const char* tkp = a.tk ? static_cast<const char*>(a.tk) + khead : kp;
  const char* tvp = a.tv ? static_cast<const char*>(a.tv) + khead : vp;
  const int64_t qbytes = int64_t(a.Nq) * a.grow;

  vec8 qB[L::NC], tqB[L::NC];
  {
    const Rsrc rq = make_rsrc(qp, qbytes), rtq = make_rsrc(tqp, a.tq ? qbytes : 0);
#pragma unroll
    for (int c = 0; c < L::NC; ++c) {
      const int col = hlf * (D / 2) + 8 * c;
      const int off = col < a.dh ? qi * a.grow + col * 2 : kOutOfRange;
      qB[c] = __builtin_bit_cast(vec8, ld128(rq, off));
      tqB[c] = __builtin_bit_cast(vec8, ld128(rtq, off));
      if constexpr (POW2) {
        qB[c] = T::scale8(qB[c], a.scale);
        tqB[c] = T::scale8(tqB[c], a.scale);
      }
    }
  }

  f32x16 accO[L::NT], accT[L::NT];
#pragma unroll
  for (int t = 0; t < L::NT; ++t) {
    accO[t] = f32x16{};
    accT[t] = f32x16{};
  }
  RowState16 st{0.0f, 0.0f, 0.0f, false};
  const Rsrc mr = mask_rsrc(a, b, h, mask_es<MASK>(2), nullptr, MASK == JVPATTN_MASK_BITS);
  const Rsrc mtr = MASK == kMaskAddT ? mask_rsrc(a, b, h, 2, a.tmask) : mr;
  auto load_mask = [&](MaskVals<MASK>& m, int k0) {
    if constexpr (MASK == kMaskAddT) mask_load_t(m, a, mr, mtr, qi, k0, hlf);
    else mask_load<MASK>(m, a, mr, qi, k0, hlf);
  };
  __shared__ int kred[2];
  int t0, t_hi;   // key tiles [t0, t_hi) may hold visible keys; loop tile k is absolute tile t0 + k
  key_tiles<T, MASK, 2>(a, mr, kred, t0, t_hi, q0, kPPBM, CAUSAL);

  const int kv_end = min(CAUSAL ? min(a.Nk, q0 + kPPBM) : a.Nk, 32 * t_hi);
  const int n_tiles = max(0, (kv_end + L::BN - 1) / L::BN - t0);
  const int last = !wave_live ? -1 : (CAUSAL ? min(n_tiles - 1, (qw0 >> 5) - t0) : n_tiles - 1);
  auto kpos = [&](int k) { return (t0 + k) * 32; };   // first key of loop tile k
  auto needs_keymask = [&](int k) { return (CAUSAL && kpos(k) + 31 > qw0) || (kpos(k) + 32 > a.Nk); };

  // Tile loads (group B only): one 16-byte slot per tensor per thread.
  const int tb = tid - 4 * 64;                     // 0..255 in group B
  const int drow = (tb & 255) >> 3, dpg = tb & 7;
  const int dlg = dpg ^ swz(drow);
  const int dl_off = dlg < (a.dh >> 3) ? drow * a.grow + (dlg << 4) : kOutOfRange;   // global, in a tile
  const int tile_g = L::BN * a.grow;
  const int64_t kbytes = int64_t(a.Nk) * a.grow;
  const Rsrc rk = make_rsrc(kp, kbytes), rv = make_rsrc(vp, kbytes);
  const Rsrc rtk = make_rsrc(tkp, a.tk ? kbytes : 0), rtv = make_rsrc(tvp, a.tv ? kbytes : 0);
  auto issue_tile = [&](int j, char* stage) {
    const int off = dl_off == kOutOfRange ? kOutOfRange : (t0 + j) * tile_g + dl_off;
    const int slot = (wave - 4) * 64 * 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)to_lds(stage + slot), 16,
                                             off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rtk, (__attribute__((address_space(3))) void*)to_lds(stage + L::TENSOR_BYTES + slot), 16, off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rv, (__attribute__((address_space(3))) void*)to_lds(stage + 2 * L::TENSOR_BYTES + slot), 16, off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rtv, (__attribute__((address_space(3))) void*)to_lds(stage + 3 * L::TENSOR_BYTES + slot), 16, off, 0, 0, 0);
  };

  int kofs[L::NC];
#pragma unroll
  for (int c = 0; c < L::NC; ++c) kofs[c] = c32 * L::ROW + (((hlf * L::NC + c) ^ swz(c32)) << 4);
  int vofs0[L::NT], vofs1[L::NT];
  {
    const int g16 = lane >> 4, i16 = lane & 15;
    const int r0 = 4 * hlf + (i16 >> 2), r1 = r0 + 8;
#pragma unroll
    for (int t = 0; t < L::NT; ++t) {
      const int gcol = 4 * t + 2 * (g16 & 1) + ((i16 & 3) >> 1);
      vofs0[t] = r0 * L::ROW + ((gcol ^ swz(r0)) << 4) + 8 * (i16 & 1);
      vofs1[t] = r1 * L::ROW + ((gcol ^ swz(r1)) << 4) + 8 * (i16 & 1);
    }
  }

  // Pipeline registers carried from a vector phase to the next matrix phase.
  vec8 ka[L::NC], tka[L::NC];          // K / dK operands of the next score products
  vec8 va[L::NT][2], tva[L::NT][2];    // V / dV operands of the next value products
  vec8 pB[2], uB[2];                   // weights of the block whose value products come next
  f32x16 sn, sdn;                      // scores of the block after that
  MaskVals<MASK> mk;                   // mask values of the block to settle next

  auto read_k = [&](const char* sb) {
#pragma unroll
    for (int c = 0; c < L::NC; ++c) {
      ka[c] = __builtin_bit_cast(vec8, lds_load<uint4>(sb, kofs[c]));
      tka[c] = __builtin_bit_cast(vec8, lds_load<uint4>(sb + L::TENSOR_BYTES, kofs[c]));
    }
  };
  auto read_v = [&](const char* sb) {
    const char* sv = sb + 2 * L::TENSOR_BYTES;
    const char* stv = sb + 3 * L::TENSOR_BYTES;
#pragma unroll
    for (int t = 0; t < L::NT; ++t)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const int o0 = 16 * kc * L::ROW + vofs0[t], o1 = 16 * kc * L::ROW + vofs1[t];
        va[t][kc] = __builtin_bit_cast(
            vec8, __builtin_shufflevector(lds_read_tr(sv + o0), lds_read_tr(sv + o1), 0, 1, 2, 3, 4, 5, 6, 7));
        tva[t][kc] = __builtin_bit_cast(
            vec8, __builtin_shufflevector(lds_read_tr(stv + o0), lds_read_tr(stv + o1), 0, 1, 2, 3, 4, 5, 6, 7));
      }
  };
  auto mma_s = [&]() {
    sn = f32x16{};
    sdn = f32x16{};
#pragma unroll
    for (int c = 0; c < L::NC; ++c) {
      sn = T::mfma(ka[c], qB[c], sn);
      sdn = T::mfma(tka[c], qB[c], sdn);
      sdn = T::mfma(ka[c], tqB[c], sdn);
    }
  };
  auto mma_v = [&]() {
#pragma unroll
    for (int t = 0; t < L::NT; ++t)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        accO[t] = T::mfma(va[t][kc], pB[kc], accO[t]);
        accT[t] = T::mfma(va[t][kc], uB[kc], accT[t]);
        accT[t] = T::mfma(tva[t][kc], pB[kc], accT[t]);
      }
  };
  // Scores of block k (in sn): mask, then weights into pB / uB. The V / dV
  // operands of block k (stage stv) are read while the weights are packed.
  auto settle = [&](int k, const char* stv) {
    // a block the mask hides from all of this wave's rows needs no softmax: its weights are zeros
    // (the value products then add nothing)
    if (MASK != JVPATTN_MASK_NONE && a.skip_hidden && !__any(mask_any_visible<T, MASK>(mk))) {
      __builtin_amdgcn_sched_barrier(0);
      read_v(stv);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        pB[kc] = vec8{};
        uB[kc] = vec8{};
      }
      return;
    }
    mask_apply<T, MASK, POW2>(sn, mk, a.scale);
    mask_tangent<T, MASK>(sdn, mk, POW2 ? 1.0f : a.inv_scale);
    if (needs_keymask(k)) hide_keys<CAUSAL>(sn, a.Nk, qi, kpos(k), hlf);
    float e[16], alpha, lsum;
    if (block_exp16<T>(sn, st, a.cx, e, alpha, lsum)) {
#pragma unroll
      for (int t = 0; t < L::NT; ++t) {
        accO[t] *= alpha;
        accT[t] *= alpha;
      }
    }
    if constexpr (__is_same(T, F16)) {
      const float shrink = f16_range_guard(e, sdn, POW2 ? 1.0f : a.scale, lsum, st.moff, st.l, st.mu);
      if (shrink != 1.0f) {
#pragma unroll
        for (int t = 0; t < L::NT; ++t) {
          accO[t] *= shrink;
          accT[t] *= shrink;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    read_v(stv);
    block_pack16<T, !POW2>(e, sdn, a.scale, pB, uB);
  };

  // Matrix phase of iteration i: value products of block i (mu takes its
  // weight products), then the score products of block i+1, whose K / dK
  // operands (stage stn) are read first so they arrive while the value
  // products run.
  auto matrix_phase = [&](int i, const char* stn) {
    if (i > last) return;
    // This wave's matrix-core instructions go ahead of the vector work of the
    // other wave on its SIMD (priority 2 against 0), so the matrix core does
    // not wait for an issue slot.
    __builtin_amdgcn_s_setprio(2);
    // On a wave's last block the score products are of no use (stn holds
    // some other tile, read harmlessly); issuing them anyway keeps the phase
    // one straight-line block the scheduler can interleave.
    read_k(stn);
    mma_v();
    block_mu16<T>(uB, st);
    mma_s();
    // The K / dK reads go out between the first value products, so their
    // issue does not hold up the matrix cores; the score products follow.
#pragma unroll
    for (int j = 0; j < 2 * L::NC; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 6 * L::NT - 2 * L::NC, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 3 * L::NC, 0);
    __builtin_amdgcn_s_setprio(0);
  };
  // Vector phase of iteration i: settle block i+1 (V / dV from stage stn).
  auto vector_phase = [&](int i, const char* stn) {
    if (i + 1 > last) return;
    settle(i + 1, stn);
    if (i + 2 <= last) load_mask(mk, kpos(i + 2));
  };
  // Group B's wait for its loads of tile j; tiles issued after j may stay in flight.
  auto wait_tile = [&](int j) {
    const int newer = min(n_tiles - 1, j + 3) - j;   // tiles issued after j so far (at most 3)
    if (newer >= 3) wait_vmcnt<12>();
    else if (newer == 2) wait_vmcnt<8>();
    else if (newer == 1) wait_vmcnt<4>();
    else wait_vmcnt<0>();
  };

  // Prologue: group B loads tiles 0..5; everyone settles block 0 and reads the
  // operands of the first matrix phase.
  if (grp_b) {
    if (n_tiles > 0) issue_tile(0, stage0);
    if (n_tiles > 1) issue_tile(1, stage1);
    if (n_tiles > 2) issue_tile(2, stage2);
    if (n_tiles > 3) issue_tile(3, stage3);
    if (n_tiles > 4) issue_tile(4, stage4);
    if (n_tiles > 5) issue_tile(5, stage5);
    const int newer = min(n_tiles - 1, 5) - 1;   // tiles issued after tile 1
    if (newer >= 4) wait_vmcnt<16>();
    else if (newer == 3) wait_vmcnt<12>();
    else if (newer == 2) wait_vmcnt<8>();
    else if (newer == 1) wait_vmcnt<4>();
    else wait_vmcnt<0>();
  }
  ring_barrier();
  if (0 <= last) {
    read_k(stage0);
    mma_s();
    load_mask(mk, kpos(0));
    settle(0, stage0);
    if (1 <= last) load_mask(mk, kpos(1));
  }
  // Operands of the first matrix phase have arrived (states the loop's entry
  // as free of pending LDS reads, as every later iteration is).
  __builtin_amdgcn_s_waitcnt(0xc07f);

  // Every wave runs matrix(i), barrier, vector(i), barrier. Group B starts
  // one barrier late, so the two waves of each SIMD are always in opposite
  // phases: A's vector(i) runs beside B's matrix(i), A's matrix(i+1) beside
  // B's vector(i). Group B loads tile i+6 into stage i%6 during matrix(i)
  // (tile i was last read in B's vector(i-1)) and waits for tile i+3 at the
  // end of vector(i) (first read in A's vector(i+1)).
  if (grp_b) {
    wait_tile(2);
    ring_barrier();
  }
  auto iteration = [&](int i, char* st_r, char* st_r1) {
    matrix_phase(i, st_r1);
    if (grp_b && i + kPPStages < n_tiles) issue_tile(i + kPPStages, st_r);
    ring_barrier();
    vector_phase(i, st_r1);
    if (grp_b) wait_tile(i + 3);
    ring_barrier();
  };
  for (int i = 0; i < n_tiles; i += kPPStages) {
    iteration(i, stage0, stage1);
    if (i + 1 < n_tiles) iteration(i + 1, stage1, stage2);
    if (i + 2 < n_tiles) iteration(i + 2, stage2, stage3);
    if (i + 3 < n_tiles) iteration(i + 3, stage3, stage4);
    if (i + 4 < n_tiles) iteration(i + 4, stage4, stage5);
    if (i + 5 < n_tiles) iteration(i + 5, stage5, stage0);
  }
  if (!grp_b) ring_barrier();

  const float l = xhalf_sum(st.l);
  const float mu = xhalf_sum(st.mu);
  if (qi < a.Nq) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const float tl = mu * inv;   // mu already sums e dS
    uint16_t* op = static_cast<uint16_t*>(a.o) + (int64_t(bh) * a.Nq + qi) * a.dh;
    uint16_t* top = static_cast<uint16_t*>(a.to) + (int64_t(bh) * a.Nq + qi) * a.dh;
#pragma unroll
    for (int t = 0; t < L::NT; ++t) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float ov[4], dv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ov[e] = accO[t][4 * g + e] * inv;
          dv[e] = accT[t][4 * g + e] * inv - tl * ov[e];
        }
        const int dd = 32 * t + 8 * g + 4 * hlf;
        if (dd < a.dh) {
          *reinterpret_cast<uint2*>(op + dd) = uint2{T::pack2(ov[0], ov[1]), T::pack2(ov[2], ov[3])};
          *reinterpret_cast<uint2*>(top + dd) = uint2{T::pack2(dv[0], dv[1]), T::pack2(dv[2], dv[3])};
        }
      }
    }
    if (hlf == 0) {
      const int64_t ri = int64_t(bh) * a.Nq + qi;
      a.lse[ri] = l > 0.0f ? (st.moff + log2f(l)) * kLn2 : -INFINITY;
      if (a.tlse) a.tlse[ri] = tl;
    }
  }
}

template <typename T, int MASK, bool CAUSAL, bool POW2>
__global__ __launch_bounds__(kPPThreads, 2) void fwd16pp_kernel(FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  fwd16pp_body<T, MASK, CAUSAL, POW2>(a);
#endif
}

// ------------------------------------------ 16-bit kernel for wide heads (d = 256)
//
// Four waves, 64 query rows: waves 2r and 2r+1 (a pair) share the 32 rows of
// row block r, and wave 2r+ch owns half ch of the head dimension, both as a
// contraction half for the scores and as the 128 output columns of O and dO
// it accumulates. Per 32-key block a wave forms its partial S and dS over its
// half, the pair swaps partials through LDS, and both add them (float32
// addition commutes, so both hold the same S and dS bit for bit and run the
// same softmax). A wave thus holds half of Q, dQ and half of the output
// accumulators, and no product is computed twice. Keys stream through a
// 2-stage LDS ring (a stage of K, dK, V, dV is 64 KB at d = 256): tile k+1 is
// fetched while block k is computed. Softmax (lazy rescale) and the value
// products are the 4-wave kernel's steps; one wave per SIMD.
constexpr int kWideBM = 64;                          // query rows per workgroup
constexpr int kWideXchg = 2 * 16 * 64 * 4;           // bytes of one wave's partial S, dS

template <typename T, int MASK, bool CAUSAL, bool POW2>
__device__ __forceinline__ void fwd16w_body(const FwdArgs& a, int t_lo, int t_hi, char* stage0, char* stage1,
                                            char* xchg) {
  constexpr int D = 256;
  using L = Tile16<D>;
  using vec8 = typename T::vec8;
  constexpr int LOADS = L::TENSOR_BYTES / (16 * kThreads);   // 16-byte loads per thread per tensor
  static_assert(LOADS * 16 * kThreads == L::TENSOR_BYTES, "tile must split evenly over the workgroup");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31;
  const int hlf = lane >> 5;

  int qb, bh;
  block_coords(a, int(blockIdx.x), qb, bh);
  const int b = bh / a.H, h = bh % a.H;
  constexpr int NT = L::NT / 2;        // accumulator tiles of this wave's column half
  const int ch = wave & 1;             // column half: output columns 128 ch .. 128 ch + 127
  const int q0 = qb * kWideBM;
  const int qw0 = q0 + 32 * (wave >> 1);
  const int qi = qw0 + c32;
  const bool wave_live = qw0 < a.Nq;

  const int64_t qhead = int64_t(bh) * a.Nq * a.grow;
  const int64_t khead = int64_t(bh / a.grp) * a.Nk * a.grow;
  const char* qp = static_cast<const char*>(a.q) + qhead;
  const char* kp = static_cast<const char*>(a.k) + khead;
  const char* vp = static_cast<const char*>(a.v) + khead;
  const char* tqp = a.tq ? static_cast<const char*>(a.tq) + qhead : qp;
  const char* tkp = a.tk ? static_cast<const char*>(a.tk) + khead : kp;
  const char* tvp = a.tv ? static_cast<const char*>(a.tv) + khead : vp;
  const int64_t qbytes = int64_t(a.Nq) * a.grow;

  constexpr int NCH = L::NC / 2;       // score chunks of this wave's contraction half
  vec8 qB[NCH], tqB[NCH];
  {
    const Rsrc rq = make_rsrc(qp, qbytes), rtq = make_rsrc(tqp, a.tq ? qbytes : 0);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int col = hlf * (D / 2) + 8 * (NCH * ch + c);
      const int off = col < a.dh ? qi * a.grow + col * 2 : kOutOfRange;
      qB[c] = __builtin_bit_cast(vec8, ld128(rq, off));
      tqB[c] = __builtin_bit_cast(vec8, ld128(rtq, off));
      if constexpr (POW2) {
        qB[c] = T::scale8(qB[c], a.scale);
        tqB[c] = T::scale8(tqB[c], a.scale);
      }
    }
  }

  f32x16 accO[NT], accT[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    accO[t] = f32x16{};
    accT[t] = f32x16{};
  }
  RowState st{-INFINITY, 0.0f, 0.0f, 0.0f};
  const Rsrc mr = mask_rsrc(a, b, h, mask_es<MASK>(2), nullptr, MASK == JVPATTN_MASK_BITS);
  const Rsrc mtr = MASK == kMaskAddT ? mask_rsrc(a, b, h, 2, a.tmask) : mr;
  const float inv_us = POW2 ? 1.0f : a.inv_scale;   // mask tangent -> units of sd

  const int kv_end = min(CAUSAL ? min(a.Nk, q0 + kWideBM) : a.Nk, 32 * t_hi);
  const int n_tiles = max(0, (kv_end + L::BN - 1) / L::BN - t_lo);
  const int last = !wave_live ? -1 : (CAUSAL ? min(n_tiles - 1, (qw0 >> 5) - t_lo) : n_tiles - 1);
  auto kpos = [&](int k) { return (t_lo + k) * 32; };
  auto needs_keymask = [&](int k) { return (CAUSAL && kpos(k) + 31 > qw0) || (kpos(k) + 32 > a.Nk); };

  int dl_off[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int p = i * kThreads + tid;
    const int row = p / L::GR, pg = p % L::GR, lg = pg ^ swz(row);
    dl_off[i] = lg < (a.dh >> 3) ? row * a.grow + (lg << 4) : kOutOfRange;
  }
  const int tile_g = L::BN * a.grow;
  const int64_t kbytes = int64_t(a.Nk) * a.grow;
  const Rsrc rk = make_rsrc(kp, kbytes), rv = make_rsrc(vp, kbytes);
  const Rsrc rtk = make_rsrc(tkp, a.tk ? kbytes : 0), rtv = make_rsrc(tvp, a.tv ? kbytes : 0);
  auto issue_tile = [&](int j, char* stage) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int off = dl_off[i] == kOutOfRange ? kOutOfRange : (t_lo + j) * tile_g + dl_off[i];
      const int slot = (i * kThreads + wave * 64) * 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)to_lds(stage + slot),
                                               16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rtk, (__attribute__((address_space(3))) void*)to_lds(stage + L::TENSOR_BYTES + slot), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rv, (__attribute__((address_space(3))) void*)to_lds(stage + 2 * L::TENSOR_BYTES + slot), 16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rtv, (__attribute__((address_space(3))) void*)to_lds(stage + 3 * L::TENSOR_BYTES + slot), 16, off, 0, 0, 0);
    }
  };

  int kofs[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) kofs[c] = c32 * L::ROW + (((hlf * L::NC + NCH * ch + c) ^ swz(c32)) << 4);
  int vofs0[NT], vofs1[NT];   // this wave's column half: 32-column tiles 4 ch .. 4 ch + 3
  {
    const int g16 = lane >> 4, i16 = lane & 15;
    const int r0 = 4 * hlf + (i16 >> 2), r1 = r0 + 8;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int gcol = 4 * (NT * ch + t) + 2 * (g16 & 1) + ((i16 & 3) >> 1);
      vofs0[t] = r0 * L::ROW + ((gcol ^ swz(r0)) << 4) + 8 * (i16 & 1);
      vofs1[t] = r1 * L::ROW + ((gcol ^ swz(r1)) << 4) + 8 * (i16 & 1);
    }
  }

  auto scores = [&](const char* sb, f32x16& s, f32x16& sd) {
    s = f32x16{};
    sd = f32x16{};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const vec8 ka = __builtin_bit_cast(vec8, lds_load<uint4>(sb, kofs[c]));
      const vec8 tka = __builtin_bit_cast(vec8, lds_load<uint4>(sb + L::TENSOR_BYTES, kofs[c]));
      s = T::mfma(ka, qB[c], s);
      sd = T::mfma(tka, qB[c], sd);
      sd = T::mfma(ka, tqB[c], sd);
    }
  };
  // partial S, dS of this wave: 8 granules of 16 bytes per lane, lane-contiguous
  char* xmine = xchg + wave * kWideXchg;
  const char* xpeer = xchg + (wave ^ 1) * kWideXchg;
  auto put_partial = [&](const f32x16& s, const f32x16& sd) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<float4*>(xmine + (j * 64 + lane) * 16) = float4{s[4 * j], s[4 * j + 1], s[4 * j + 2], s[4 * j + 3]};
      *reinterpret_cast<float4*>(xmine + ((4 + j) * 64 + lane) * 16) =
          float4{sd[4 * j], sd[4 * j + 1], sd[4 * j + 2], sd[4 * j + 3]};
    }
  };
  auto add_peer = [&](f32x16& s, f32x16& sd) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 ps = *reinterpret_cast<const float4*>(xpeer + (j * 64 + lane) * 16);
      const float4 pd = *reinterpret_cast<const float4*>(xpeer + ((4 + j) * 64 + lane) * 16);
      s[4 * j] += ps.x;
      s[4 * j + 1] += ps.y;
      s[4 * j + 2] += ps.z;
      s[4 * j + 3] += ps.w;
      sd[4 * j] += pd.x;
      sd[4 * j + 1] += pd.y;
      sd[4 * j + 2] += pd.z;
      sd[4 * j + 3] += pd.w;
    }
  };
  // Value products. A pending rescale of the accumulators (alpha, when rs) is
  // applied tile by tile just before that tile's products: scaled in one
  // place, all 128 accumulator registers would be copied out of the AGPRs at
  // once. The flag goes through an empty asm per tile so that the compiler
  // keeps the four conditional blocks apart.
  auto values = [&](const char* sb, const vec8 (&pB)[2], const vec8 (&uB)[2], bool rs, float alpha) {
    const char* sv = sb + 2 * L::TENSOR_BYTES;
    const char* stv = sb + 3 * L::TENSOR_BYTES;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      int rst = __builtin_amdgcn_readfirstlane(static_cast<int>(rs));
      asm volatile("" : "+s"(rst));
      if (rst) {
        accO[t] *= alpha;
        accT[t] *= alpha;
      }
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const int o0 = 16 * kc * L::ROW + vofs0[t], o1 = 16 * kc * L::ROW + vofs1[t];
        const vec8 va = __builtin_bit_cast(
            vec8, __builtin_shufflevector(lds_read_tr(sv + o0), lds_read_tr(sv + o1), 0, 1, 2, 3, 4, 5, 6, 7));
        const vec8 tva = __builtin_bit_cast(
            vec8, __builtin_shufflevector(lds_read_tr(stv + o0), lds_read_tr(stv + o1), 0, 1, 2, 3, 4, 5, 6, 7));
        accO[t] = T::mfma(va, pB[kc], accO[t]);
        accT[t] = T::mfma(va, uB[kc], accT[t]);
        accT[t] = T::mfma(tva, pB[kc], accT[t]);
      }
    }
  };

  // Every wave passes both barriers of every iteration (the pairs' row blocks
  // differ in causal extent and in mask visibility); the two waves of a pair
  // take the same branches, as they read the same rows.
  if (n_tiles > 0) issue_tile(0, stage0);
  for (int k = 0; k < n_tiles; ++k) {
    char* cur = (k & 1) ? stage1 : stage0;
    char* nxt = (k & 1) ? stage0 : stage1;
    wait_vmcnt<0>();   // this thread's loads of tile k
    ring_barrier();    // tile k visible to all; every wave is done with tile k-1 (stage nxt) and its swap
    if (k + 1 < n_tiles) issue_tile(k + 1, nxt);
    bool live = k <= last;
    MaskVals<MASK> mk;
    if (live) {
      if constexpr (MASK == kMaskAddT) mask_load_t(mk, a, mr, mtr, qi, kpos(k), hlf);
      else mask_load<MASK>(mk, a, mr, qi, kpos(k), hlf);
      if (MASK != JVPATTN_MASK_NONE && a.skip_hidden && !__any(mask_any_visible<T, MASK>(mk))) live = false;
    }
    f32x16 s, sd;
    if (live) {
      scores(cur, s, sd);
      put_partial(s, sd);
    }
    ring_barrier();    // both partials of each pair in LDS
    if (!live) continue;
    add_peer(s, sd);
    mask_apply<T, MASK, POW2>(s, mk, a.scale);
    mask_tangent<T, MASK>(sd, mk, inv_us);
    if (needs_keymask(k)) hide_keys<CAUSAL>(s, a.Nk, qi, kpos(k), hlf);
    float alpha;
    bool rs = update_max(block_max(s), st, a.cx, a.thr, alpha);
    const float lsum = exp_l(s, st, a.cx);
    if constexpr (__is_same(T, F16)) {
      const float moff0 = st.moff;
      const float shrink = f16_range_guard(s, sd, POW2 ? 1.0f : a.scale, lsum, st.moff, st.l, st.mu);
      if (shrink != 1.0f) st.m += (st.moff - moff0) / a.cx;
      alpha *= shrink;                    // alpha and shrink are 1 on lanes that keep their scale
      rs = rs || __any(shrink != 1.0f);   // uniform over the wave, like update_max's result
    }
    float u[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) u[r] = POW2 ? sd[r] * s[r] : (sd[r] * a.scale) * s[r];
    st.mu += sum16(u);
    vec8 pB[2], uB[2];
    {
      uint32_t pw[8], uw[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pw[i] = T::pack2(s[2 * i], s[2 * i + 1]);
        uw[i] = T::pack2(u[2 * i], u[2 * i + 1]);
      }
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        pB[kc] = __builtin_bit_cast(vec8, uint4{pw[4 * kc], pw[4 * kc + 1], pw[4 * kc + 2], pw[4 * kc + 3]});
        uB[kc] = __builtin_bit_cast(vec8, uint4{uw[4 * kc], uw[4 * kc + 1], uw[4 * kc + 2], uw[4 * kc + 3]});
      }
    }
    values(cur, pB, uB, rs, alpha);
  }

  const float l = xhalf_sum(st.l);
  const float mu = xhalf_sum(st.mu);
  if (qi < a.Nq) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const float tl = mu * inv;   // mu sums e dS (float32 products)
    uint16_t* op = static_cast<uint16_t*>(a.o) + (int64_t(bh) * a.Nq + qi) * a.dh;
    uint16_t* top = static_cast<uint16_t*>(a.to) + (int64_t(bh) * a.Nq + qi) * a.dh;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float ov[4], dv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ov[e] = accO[t][4 * g + e] * inv;
          dv[e] = accT[t][4 * g + e] * inv - tl * ov[e];
        }
        const int dd = 32 * (NT * ch + t) + 8 * g + 4 * hlf;
        if (dd < a.dh) {
          *reinterpret_cast<uint2*>(op + dd) = uint2{T::pack2(ov[0], ov[1]), T::pack2(ov[2], ov[3])};
          *reinterpret_cast<uint2*>(top + dd) = uint2{T::pack2(dv[0], dv[1]), T::pack2(dv[2], dv[3])};
        }
      }
    }
    if (hlf == 0 && ch == 0) {   // both waves of the pair hold the same row statistics
      const int64_t ri = int64_t(bh) * a.Nq + qi;
      a.lse[ri] = l > 0.0f ? (st.moff + log2f(l)) * kLn2 : -INFINITY;
      if (a.tlse) a.tlse[ri] = tl;
    }
  }
}

template <typename T, int MASK, bool CAUSAL, bool POW2>
__global__ __launch_bounds__(kThreads, 1) void fwd16w_kernel(FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using L = Tile16<256>;
  // 2 x 64 KB ring + 4 x 8 KB partials: the whole 160 KB of a CU's LDS, so the
  // key-range scratch of key_tiles lives in the partials' space (it is read
  // before the first ring barrier, and the partials are written after it)
  static_assert(2 * L::STAGE_BYTES + 4 * kWideXchg <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) char smem[2 * L::STAGE_BYTES + 4 * kWideXchg];
  char* xchg = smem + 2 * L::STAGE_BYTES;
  int t_lo, t_hi;
  {
    int qb, bh;
    block_coords(a, int(blockIdx.x), qb, bh);
    const Rsrc mr = mask_rsrc(a, bh / a.H, bh % a.H, mask_es<MASK>(2), nullptr, MASK == JVPATTN_MASK_BITS);
    key_tiles<T, MASK, 2>(a, mr, reinterpret_cast<int*>(xchg), t_lo, t_hi, qb * kWideBM, kWideBM, CAUSAL);
  }
  fwd16w_body<T, MASK, CAUSAL, POW2>(a, t_lo, t_hi, smem, smem + L::STAGE_BYTES, xchg);
#endif
}

// ------------------------------------------------------------- float32 kernel
//
// Same structure on v_mfma_f32_32x32x2_f32 (float32 products, no rounding of
// the weights). Each product takes 2 entries of the inner dimension: for the
// score products lane half hlf supplies head-dim entry hlf*D/2 + i for
// product i; for the value products, product m contracts over the keys held
// in C register m of each lane half, so P^T and (P dS)^T are used as they are.


template <int D, int MASK, bool CAUSAL>
__device__ __forceinline__ void fwd32_body(const FwdArgs& a) {
  using L = Tile32<D>;
  extern __shared__ __attribute__((aligned(16))) char smem32[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c32 = lane & 31;
  const int hlf = lane >> 5;

  int qb, bh;
  block_coords(a, int(blockIdx.x), qb, bh);
  const int b = bh / a.H, h = bh % a.H;
  const int q0 = qb * kBM;
  const int qw0 = q0 + 32 * wave;
  const int qi = qw0 + c32;
  const bool wave_live = qw0 < a.Nq;

  // global rows hold a.dh <= D logical columns; the others read as zeros and are never stored
  const float* qp = static_cast<const float*>(a.q) + int64_t(bh) * a.Nq * a.dh;
  const float* tqp = a.tq ? static_cast<const float*>(a.tq) + int64_t(bh) * a.Nq * a.dh : nullptr;
  const int64_t khead = int64_t(bh / a.grp) * a.Nk * a.dh;   // the key/value head it reads
  const float* kp = static_cast<const float*>(a.k) + khead;
  const float* vp = static_cast<const float*>(a.v) + khead;
  const float* tkp = a.tk ? static_cast<const float*>(a.tk) + khead : nullptr;
  const float* tvp = a.tv ? static_cast<const float*>(a.tv) + khead : nullptr;

  float qB[D / 2], tqB[D / 2];
  {
#pragma unroll
    for (int i = 0; i < D / 2; i += 4) {
      const bool ok = qi < a.Nq && hlf * (D / 2) + i < a.dh;
      const int64_t off = int64_t(qi) * a.dh + hlf * (D / 2) + i;
      f32x4 x = ok ? *reinterpret_cast<const f32x4*>(qp + off) : f32x4{};
      f32x4 y = (ok && tqp) ? *reinterpret_cast<const f32x4*>(tqp + off) : f32x4{};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qB[i + e] = x[e];
        tqB[i + e] = y[e];
      }
    }
  }

  f32x16 accO[L::NT], accT[L::NT];
#pragma unroll
  for (int t = 0; t < L::NT; ++t) {
    accO[t] = f32x16{};
    accT[t] = f32x16{};
  }
  RowState st{-INFINITY, 0.0f, 0.0f, 0.0f};
  const Rsrc mr = mask_rsrc(a, b, h, mask_es<MASK>(4), nullptr, MASK == JVPATTN_MASK_BITS);
  const Rsrc mtr = MASK == kMaskAddT ? mask_rsrc(a, b, h, 4, a.tmask) : mr;
  __shared__ int kred[2];
  int t0, t_hi;   // key tiles [t0, t_hi) may hold visible keys
  key_tiles<F16, MASK, 4>(a, mr, kred, t0, t_hi, q0, kBM, CAUSAL);

  const int kv_end = min(CAUSAL ? min(a.Nk, q0 + kBM) : a.Nk, 32 * t_hi);
  const int n_tiles = max(0, (kv_end + L::BN - 1) / L::BN - t0);
  char* sk = smem32;
  char* stk = smem32 + L::TENSOR_BYTES;
  char* sv = smem32 + 2 * L::TENSOR_BYTES;
  char* stv = smem32 + 3 * L::TENSOR_BYTES;

  for (int j = 0; j < n_tiles; ++j) {
    const int kbase = (t0 + j) * L::BN;
    // Global -> LDS. K rows as granules; V transposed element by element.
    for (int gi = tid; gi < L::BN * L::GR; gi += kThreads) {
      const int row = gi / L::GR, g = gi % L::GR;
      const int key = kbase + row;
      const int64_t off = int64_t(key) * a.dh + 4 * g;
      const bool ok = key < a.Nk && 4 * g < a.dh;
      lds_store<f32x4>(sk, k32_off<D>(row, g), ok ? *reinterpret_cast<const f32x4*>(kp + off) : f32x4{});
      lds_store<f32x4>(stk, k32_off<D>(row, g),
                       (ok && tkp) ? *reinterpret_cast<const f32x4*>(tkp + off) : f32x4{});
      const f32x4 x = ok ? *reinterpret_cast<const f32x4*>(vp + off) : f32x4{};
      const f32x4 y = (ok && tvp) ? *reinterpret_cast<const f32x4*>(tvp + off) : f32x4{};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int dd = 4 * g + e;
        const int voff = vt32_off(dd, row >> 2) + 4 * (row & 3);
        lds_store<float>(sv, voff, x[e]);
        lds_store<float>(stv, voff, y[e]);
      }
    }
    __syncthreads();

    const int k0 = kbase;
    if (wave_live && k0 < kv_end && !(CAUSAL && k0 > qw0 + 31)) {
      f32x16 s{}, sd{};
#pragma unroll
      for (int i = 0; i < D / 2; i += 4) {
        const int g = (hlf * (D / 2) + i) / 4;
        const f32x4 ka = lds_load<f32x4>(sk, k32_off<D>(c32, g));
        const f32x4 tka = lds_load<f32x4>(stk, k32_off<D>(c32, g));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s = __builtin_amdgcn_mfma_f32_32x32x2f32(ka[e], qB[i + e], s, 0, 0, 0);
          sd = __builtin_amdgcn_mfma_f32_32x32x2f32(tka[e], qB[i + e], sd, 0, 0, 0);
          sd = __builtin_amdgcn_mfma_f32_32x32x2f32(ka[e], tqB[i + e], sd, 0, 0, 0);
        }
      }
      const bool elem_mask = (CAUSAL && k0 + 31 > qw0) || (k0 + 32 > a.Nk);
      constexpr bool ADD = MASK == JVPATTN_MASK_ADDITIVE || MASK == kMaskAddT;
      mask_scores<F16, ADD ? -1 : MASK, CAUSAL, false>(s, a, mr, qi, k0, hlf, elem_mask);
      if constexpr (ADD) {
        // float32 additive mask: element (qi, key) for the 16 keys of this lane
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + (r >> 2) * 8 + 4 * hlf + (r & 3);
          const float mv = __uint_as_float(
              __builtin_amdgcn_raw_buffer_load_b32(mr, (qi * int(a.msq) + key) * 4, 0, 0));
          s[r] = fmaf(s[r], a.scale, mv);   // hidden keys are already -inf
          if constexpr (MASK == kMaskAddT) {
            // the mask's tangent joins the score tangent (sd * scale = dS)
            const float tv = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(mtr, (qi * int(a.msq) + key) * 4, 0, 0));
            sd[r] = fmaf(tv, a.inv_scale, sd[r]);
          }
        }
      }
      float alpha;
      if (softmax_block(s, sd, st, a.cx, a.thr, alpha)) {
#pragma unroll
        for (int t = 0; t < L::NT; ++t) {
          accO[t] *= alpha;
          accT[t] *= alpha;
        }
      }
#pragma unroll
      for (int t = 0; t < L::NT; ++t) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int off = vt32_off(32 * t + c32, 2 * g + hlf);
          const f32x4 va = lds_load<f32x4>(sv, off);
          const f32x4 tva = lds_load<f32x4>(stv, off);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int m = 4 * g + e;
            accO[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(va[e], s[m], accO[t], 0, 0, 0);
            accT[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(va[e], sd[m] * a.scale, accT[t], 0, 0, 0);
            accT[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(tva[e], s[m], accT[t], 0, 0, 0);
          }
        }
      }
    }
    __syncthreads();
  }

  const float l = xhalf_sum(st.l);
  const float mu = xhalf_sum(st.mu);
  if (qi < a.Nq) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const float tl = mu * a.scale * inv;
    float* op = static_cast<float*>(a.o) + (int64_t(bh) * a.Nq + qi) * a.dh;
    float* top = static_cast<float*>(a.to) + (int64_t(bh) * a.Nq + qi) * a.dh;
#pragma unroll
    for (int t = 0; t < L::NT; ++t) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 ov, dv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ov[e] = accO[t][4 * g + e] * inv;
          dv[e] = accT[t][4 * g + e] * inv - tl * ov[e];
        }
        const int dd = 32 * t + 8 * g + 4 * hlf;
        if (dd < a.dh) {
          *reinterpret_cast<f32x4*>(op + dd) = ov;
          *reinterpret_cast<f32x4*>(top + dd) = dv;
        }
      }
    }
    if (hlf == 0) {
      const int64_t ri = int64_t(bh) * a.Nq + qi;
      a.lse[ri] = l > 0.0f ? (st.moff + log2f(l)) * kLn2 : -INFINITY;
      if (a.tlse) a.tlse[ri] = tl;
    }
  }
}

template <int D, int MASK, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd32_kernel(FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  fwd32_body<D, MASK, CAUSAL>(a);
#endif
}

// ---------------------------------------------------------------- dispatch

// The 4-wave kernel for d = 64: whole key range (split = 0), or halves over
// two groups of four waves (split = 1). Halves over two groups of two waves on
// 64-row blocks (split = 2) go to launch_fwd_split64.
template <typename T, int MASK, bool CAUSAL, bool POW2>
void launch_d64(int split, const FwdArgs& args, dim3 grid, hipStream_t stream) {
  if (split == 1)
    hipLaunchKernelGGL((fwd16_kernel<T, 64, MASK, CAUSAL, POW2, 2, 4>), grid, dim3(2 * kThreads), 0, stream, args);
  else
    hipLaunchKernelGGL((fwd16_kernel<T, 64, MASK, CAUSAL, POW2, 1, 4>), grid, dim3(kThreads), 0, stream, args);
}

template <int MASK, bool CAUSAL>
hipError_t launch_typed(int dtype, int d, bool pow2, int split, const FwdArgs& args, dim3 grid,
                        hipStream_t stream) {
  const dim3 block(kThreads);
  if (d == 256) return launch_fwd_d256<MASK, CAUSAL>(dtype, pow2, args, grid, stream);  // 16-bit only
  if (d == 64 && split == 2 && dtype != JVPATTN_F32)
    return launch_fwd_split64<MASK, CAUSAL>(dtype, pow2, args, grid, stream);
  if (d == 128 && dtype != JVPATTN_F32) return launch_fwd_d128<MASK, CAUSAL>(dtype, pow2, args, grid, stream);
  if (dtype == JVPATTN_BF16) {
    if (pow2) launch_d64<BF16, MASK, CAUSAL, true>(split, args, grid, stream);
    else launch_d64<BF16, MASK, CAUSAL, false>(split, args, grid, stream);
  } else if (dtype == JVPATTN_F16) {
    if (pow2) launch_d64<F16, MASK, CAUSAL, true>(split, args, grid, stream);
    else launch_d64<F16, MASK, CAUSAL, false>(split, args, grid, stream);
  } else {
    if (d == 64) {
      hipLaunchKernelGGL((fwd32_kernel<64, MASK, CAUSAL>), grid, block, Tile32<64>::BUF_BYTES, stream, args);
    } else {
      auto fn = fwd32_kernel<128, MASK, CAUSAL>;
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         Tile32<128>::BUF_BYTES);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(fn, grid, block, Tile32<128>::BUF_BYTES, stream, args);
    }
  }
  return hipGetLastError();
}

}  // namespace

#if defined(JVPATTN_INST_FAMILY) && JVPATTN_INST_FAMILY == 4
template <int MASK, bool CAUSAL>
hipError_t launch_fwd_d256(int dtype, bool pow2, const FwdArgs& args, dim3 grid, hipStream_t stream) {
  const dim3 block(kThreads);
  if (dtype == JVPATTN_BF16) {
    if (pow2) hipLaunchKernelGGL((fwd16w_kernel<BF16, MASK, CAUSAL, true>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((fwd16w_kernel<BF16, MASK, CAUSAL, false>), grid, block, 0, stream, args);
  } else {
    if (pow2) hipLaunchKernelGGL((fwd16w_kernel<F16, MASK, CAUSAL, true>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((fwd16w_kernel<F16, MASK, CAUSAL, false>), grid, block, 0, stream, args);
  }
  return hipGetLastError();
}
#endif

#if defined(JVPATTN_INST_FAMILY) && JVPATTN_INST_FAMILY == 3
template <int MASK, bool CAUSAL>
hipError_t launch_fwd_d128(int dtype, bool pow2, const FwdArgs& args, dim3 grid, hipStream_t stream) {
  const dim3 block(kThreads);
  if (dtype == JVPATTN_BF16) {
    if (pow2) hipLaunchKernelGGL((fwd16_kernel<BF16, 128, MASK, CAUSAL, true, 1, 4>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((fwd16_kernel<BF16, 128, MASK, CAUSAL, false, 1, 4>), grid, block, 0, stream, args);
  } else {
    if (pow2) hipLaunchKernelGGL((fwd16_kernel<F16, 128, MASK, CAUSAL, true, 1, 4>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((fwd16_kernel<F16, 128, MASK, CAUSAL, false, 1, 4>), grid, block, 0, stream, args);
  }
  return hipGetLastError();
}
#endif

#if defined(JVPATTN_INST_FAMILY) && JVPATTN_INST_FAMILY == 2
template <int MASK, bool CAUSAL>
hipError_t launch_fwd_pp(int dtype, bool pow2, const FwdArgs& args, dim3 grid, hipStream_t stream) {
  const dim3 block(kPPThreads);
  if (dtype == JVPATTN_BF16) {
    if (pow2) hipLaunchKernelGGL((fwd16pp_kernel<BF16, MASK, CAUSAL, true>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((fwd16pp_kernel<BF16, MASK, CAUSAL, false>), grid, block, 0, stream, args);
  } else {
    if (pow2) hipLaunchKernelGGL((fwd16pp_kernel<F16, MASK, CAUSAL, true>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((fwd16pp_kernel<F16, MASK, CAUSAL, false>), grid, block, 0, stream, args);
  }
  return hipGetLastError();
}
#endif

#if defined(JVPATTN_INST_FAMILY) && JVPATTN_INST_FAMILY == 1
template <int MASK, bool CAUSAL>
hipError_t launch_fwd_split64(int dtype, bool pow2, const FwdArgs& args, dim3 grid, hipStream_t stream) {
  const dim3 block(2 * 128);
  if (dtype == JVPATTN_BF16) {
    if (pow2) hipLaunchKernelGGL((fwd16_kernel<BF16, 64, MASK, CAUSAL, true, 2, 2>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((fwd16_kernel<BF16, 64, MASK, CAUSAL, false, 2, 2>), grid, block, 0, stream, args);
  } else {
    if (pow2) hipLaunchKernelGGL((fwd16_kernel<F16, 64, MASK, CAUSAL, true, 2, 2>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((fwd16_kernel<F16, 64, MASK, CAUSAL, false, 2, 2>), grid, block, 0, stream, args);
  }
  return hipGetLastError();
}
#endif

// Launch the forward kernel `kernel` (FwdKernel) for this mask kind and causal
// flag; the element type, head dimension and power-of-two scale select the
// instance. Arguments were validated and planned by the caller.
template <int MASK, bool CAUSAL>
hipError_t launch_fwd(int kernel, int dtype, int d, bool pow2, const FwdArgs& args, dim3 grid, hipStream_t stream) {
  if (kernel == kFwdPingPong) return launch_fwd_pp<MASK, CAUSAL>(dtype, pow2, args, grid, stream);
  const int split = kernel == kFwdSplit ? 1 : kernel == kFwdSplit64 ? 2 : 0;
  return launch_typed<MASK, CAUSAL>(dtype, d, pow2, split, args, grid, stream);
}

}  // namespace jvpattn
