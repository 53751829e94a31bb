// Launch interface between the forward's host planner (jvpattn_fwd.hip) and
// the kernel instances (jvpattn_fwd_inst.hip, one object per mask kind and
// causal flag). Host and device code.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace jvpattn {

// Internal mask kind: an additive mask together with its tangent dM, which
// the score tangent gains (dS = scale (dQ K^T + Q dK^T) + dM).
constexpr int kMaskAddT = 4;   // beyond the public jvpattn_mask_kind values

// Lazy-rescale thresholds of the 4-wave and float32 kernels, in log2 units:
// weights may grow to 2^tau before the reference maximum moves. float16
// keeps them <= 2^4 so that weights times score tangents stay below 65504.
constexpr float kTauBF16 = 8.0f, kTauF16 = 4.0f, kTauF32 = 8.0f;

// Kernel families of the 16-bit forward (float32 has one kernel of its own);
// the values are the public jvpattn_fwd_kernel ones.
enum FwdKernel {
  kFwdWG4 = 0,        // 4 waves, 128 query rows per workgroup
  kFwdPingPong = 1,   // 8 waves in two alternating groups, 256 rows (d = 64)
  kFwdSplit = 2,      // the 4-wave body, key range split over two groups of 4 waves (d = 64)
  kFwdSplit64 = 3,    // the same on 64-row blocks, two groups of 2 waves (d = 64)
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* tq;
  const void* tk;
  const void* tv;
  const void* mask;
  const void* tmask;  // tangent of the additive mask (mask kind kMaskAddT), laid out as the mask
  void* o;
  void* to;
  float* lse;
  float* tlse;
  int H, Nq, Nk, BH;
  int dh;             // logical head dimension (columns of every global row)
  int grow;           // bytes of one global row: dh * element size
  int grp;            // query heads per key/value head (grouped-query attention; 1 = one each)
  int xgrp;           // grp when whole key/value groups can be kept on one XCD, else 1
  int head_major;     // 1: the query blocks of a head run back to back on one XCD (large grids)
  int key_range;      // 1: the mask is shared by all query rows; skip 32-key tiles it hides entirely
  int skip_hidden;    // 1: a wave skips the softmax and value products of a block its mask hides entirely
  int row_range;      // 1: one mask row per query; run only the key tiles visible to some row of the workgroup
  int n_qblk;
  int n_items;        // row blocks in all (n_qblk * BH); the mask-free 4-wave kernel walks them with a
                      // grid that may be smaller
  int mask_vec;       // 1: mask rows may be read 4 keys at a time
  int64_t msb, msh, msq;
  float scale;
  float inv_scale;    // 1 / scale
  float cx;           // score units -> log2 units
  float thr;          // lazy-rescale threshold in score units
};

template <int MASK, bool CAUSAL>
hipError_t launch_fwd(int kernel, int dtype, int d, bool pow2, const FwdArgs& args, dim3 grid, hipStream_t stream);

// The 64-row split kernel (d = 64, 16-bit: two groups of two waves), which
// launch_fwd hands over to; built in objects of its own, one per mask kind and
// causal flag, so that they can take compiler flags of their own.
template <int MASK, bool CAUSAL>
hipError_t launch_fwd_split64(int dtype, bool pow2, const FwdArgs& args, dim3 grid, hipStream_t stream);

// The ping-pong kernel (d = 64, 16-bit), the 4-wave kernel at width 128
// (d = 96 / 128, 16-bit) and the d = 256 kernel (16-bit), likewise in objects
// of their own.
template <int MASK, bool CAUSAL>
hipError_t launch_fwd_pp(int dtype, bool pow2, const FwdArgs& args, dim3 grid, hipStream_t stream);
template <int MASK, bool CAUSAL>
hipError_t launch_fwd_d128(int dtype, bool pow2, const FwdArgs& args, dim3 grid, hipStream_t stream);
template <int MASK, bool CAUSAL>
hipError_t launch_fwd_d256(int dtype, bool pow2, const FwdArgs& args, dim3 grid, hipStream_t stream);

}  // namespace jvpattn
