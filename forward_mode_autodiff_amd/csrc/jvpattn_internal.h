// Declarations shared by the validator and the launcher (host code only).
#pragma once

#include <cstddef>
#include <cstdint>

#include "jvpattn.h"

namespace jvpattn {

struct FwdSizes {
  int64_t rows_q = 0;   // B*H*Nq
  int64_t rows_k = 0;   // B*Hkv*Nk
  int elem_bytes = 0;
  int hkv = 0;          // key/value heads (params->Hkv, 0 read as H)
  int group = 1;        // query heads per key/value head, H / hkv
};

int elem_bytes(int dtype);

// Full argument check of jvpattn_fwd; fills `sizes` on success (may be NULL).
int check_fwd(const jvpattn_params* p, const void* q, const void* k, const void* v,
              const void* tq, const void* tk, const void* tv, const void* mask,
              const void* o, const void* to, const float* lse, const float* tlse,
              FwdSizes* sizes);

// check_fwd, then the additive mask's tangent tmask (NULL = zero): only with an
// additive mask, aligned to the element size, disjoint from the outputs.
int check_fwd_tmask(const jvpattn_params* p, const void* q, const void* k, const void* v,
                    const void* tq, const void* tk, const void* tv, const void* mask, const void* tmask,
                    const void* o, const void* to, const float* lse, const float* tlse, FwdSizes* sizes);

// Full argument check of jvpattn_bwd (the forward's checks on the shared
// arguments, then its own); fills `sizes` on success (may be NULL).
int check_bwd(const jvpattn_params* p, const void* q, const void* k, const void* v,
              const void* tq, const void* tk, const void* tv, const void* mask,
              const void* o, const void* to, const float* lse, const float* tlse,
              const void* go, const void* gto, const void* dq, const void* dk, const void* dv,
              const void* dtq, const void* dtk, const void* dtv, const void* workspace,
              size_t workspace_bytes, FwdSizes* sizes);

// check_bwd, then the additive mask's tangent as check_fwd_tmask checks it,
// also disjoint from the gradients and the workspace.
int check_bwd_tmask(const jvpattn_params* p, const void* q, const void* k, const void* v,
                    const void* tq, const void* tk, const void* tv, const void* mask, const void* tmask,
                    const void* o, const void* to, const float* lse, const float* tlse,
                    const void* go, const void* gto, const void* dq, const void* dk, const void* dv,
                    const void* dtq, const void* dtk, const void* dtv, const void* workspace,
                    size_t workspace_bytes, FwdSizes* sizes);

// HIP error of the most recent JVPATTN_ERR_HIP on this thread (jvpattn_last_hip_error).
extern thread_local int g_last_hip_error;

// Workspace of jvpattn_bwd: four float32 arrays of B*H*Nq (see jvpattn_bwd.hip).
int64_t bwd_workspace_bytes(int64_t rows_q);

// Compute units of the current device (queried once per device), or 0.
int cu_count();

// Grid of the kernels that walk their blocks (several per workgroup): the
// cap set by jvpattn_set_workgroups, else one workgroup per CU of the current
// device; rounded down to a multiple of 8 (so each workgroup keeps its XCD)
// when at least 8; 0 if unknown (then every block gets its own workgroup).
int walk_workgroups();

}  // namespace jvpattn
