// Declarations shared by the validator and the launcher (host code only).
#pragma once

#include <cstdint>

#include "jvpattn.h"

namespace jvpattn {

struct FwdSizes {
  int64_t rows_q = 0;   // B*H*Nq
  int64_t rows_k = 0;   // B*H*Nk
  int elem_bytes = 0;
};

int elem_bytes(int dtype);

// Full argument check of jvpattn_fwd; fills `sizes` on success (may be NULL).
int check_fwd(const jvpattn_params* p, const void* q, const void* k, const void* v,
              const void* tq, const void* tk, const void* tv, const void* mask,
              const void* o, const void* to, const float* lse, const float* tlse,
              FwdSizes* sizes);

}  // namespace jvpattn
