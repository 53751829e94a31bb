// Reverse pass: the argument block of its kernels and their launchers. The
// kernels are instantiated per head dimension and per side (keys / queries)
// in jvpattn_bwd_inst.hip, so those objects build in parallel; the host side
// (jvpattn_bwd.hip) fills the arguments and calls the launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "jvpattn.h"

namespace jvpattn {

constexpr int kBWaves = 4;
constexpr int kBThreads = 64 * kBWaves;
constexpr int kBBlk = 32 * kBWaves;   // keys (dkv) or queries (dq) per workgroup

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* tq;
  const void* tk;
  const void* tv;
  const void* mask;
  const void* tmask;  // tangent of the additive mask (kind kMaskAddT), laid out as the mask
  const void* o;
  const void* to;
  const void* go;
  const void* gto;
  const float* lse;
  const float* tlse;
  void* dq;
  void* dk;
  void* dv;
  void* dtq;
  void* dtk;
  void* dtv;
  float* ws;          // [4][ws_stride]: -lse*log2e, tlse, r, del
  int64_t ws_stride;  // floats per workspace array
  int H, Nq, Nk, BH;
  int grp;            // query heads per key/value head (grouped-query attention; 1 = one each)
  int BHK;            // key/value heads in all: B * H / grp
  int n_blk;
  int n_items;        // key-side items (key blocks x K/V heads) the walking dkv kernel covers
  int max_wgs;        // grid of a walking kernel (0: one workgroup per item)
  int dq_two;         // d = 64: the query side without its pipeline, two workgroups per CU
  int mask_vec;
  int64_t msb, msh, msq;
  float scale;
  float inv_scale;    // 1 / scale
  float cx;           // score units -> log2 units
};

enum { WS_NEGL = 0, WS_TLSE = 1, WS_R = 2, WS_DEL = 3 };

// Queue the kernels of head dimension D (64 or 128) for validated
// arguments: WHICH = kLaunchRows the rows kernel (per-row statistics into the
// workspace), kLaunchDkv the key-side gradients, kLaunchDq the query-side
// ones. Both sides read the workspace the rows kernel writes and nothing
// else the other writes, so they may run in either order or at once once it
// is done. mask_kind may be kMaskAddT (an additive mask with a tangent);
// pow2: the scale is a power of two (folded into Q, K exactly in bfloat16).
enum { kLaunchDkv = 0, kLaunchDq = 1, kLaunchRows = 2 };
template <int WHICH, int D>
hipError_t bwd_launch_part(const BwdArgs& a, int64_t rows_q, jvpattn_dtype dtype, int mask_kind, bool causal,
                           bool pow2, hipStream_t s);

}  // namespace jvpattn
