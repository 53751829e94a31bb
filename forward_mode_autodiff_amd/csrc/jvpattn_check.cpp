// Host-side argument validation for jvpattn_fwd. Pure C++: no HIP calls and
// no pointer dereferences, so it runs (and is tested) on machines without a
// GPU and under host sanitizers.
#include "jvpattn.h"
#include "jvpattn_internal.h"

#include <cmath>
#include <cstdint>

namespace jvpattn {

namespace {

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
  bool empty() const { return hi <= lo; }
};

Span span(const void* p, int64_t bytes) {
  uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Span{a, p ? a + static_cast<uintptr_t>(bytes) : a};
}

bool overlap(Span a, Span b) {
  if (a.empty() || b.empty()) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

int elem_bytes(int dtype) {
  switch (dtype) {
    case JVPATTN_F32: return 4;
    case JVPATTN_F16: return 2;
    case JVPATTN_BF16: return 2;
    default: return 0;
  }
}

int check_fwd(const jvpattn_params* p, const void* q, const void* k, const void* v,
              const void* tq, const void* tk, const void* tv, const void* mask,
              const void* o, const void* to, const float* lse, const float* tlse,
              FwdSizes* sizes) {
  if (!p) return JVPATTN_ERR_NULL;
  const int es = elem_bytes(p->dtype);
  if (es == 0) return JVPATTN_ERR_DTYPE;
  if (p->B < 0 || p->H < 0 || p->Nq < 0 || p->Nk < 0 || p->d <= 0) return JVPATTN_ERR_SHAPE;
  // grouped key/value heads: Hkv divides H (0 stands for H)
  const int hkv = p->Hkv == 0 ? p->H : p->Hkv;
  if (hkv < 0 || hkv > p->H || (hkv == 0) != (p->H == 0) || (hkv > 0 && p->H % hkv != 0))
    return JVPATTN_ERR_SHAPE;

  int64_t bh, bhk, rows_q, rows_k, n_q, n_k, bytes_q, bytes_k, bytes_stats;
  if (!mul_ok(p->B, p->H, &bh) || !mul_ok(p->B, hkv, &bhk) || !mul_ok(bh, p->Nq, &rows_q) ||
      !mul_ok(bhk, p->Nk, &rows_k) ||
      !mul_ok(rows_q, p->d, &n_q) || !mul_ok(rows_k, p->d, &n_k) || !mul_ok(n_q, es, &bytes_q) ||
      !mul_ok(n_k, es, &bytes_k) || !mul_ok(rows_q, 4, &bytes_stats))
    return JVPATTN_ERR_SHAPE;
  // every grid dimension the launcher forms must stay within int32
  if (bh > INT32_MAX) return JVPATTN_ERR_SHAPE;

  if (p->d != 32 && p->d != 64 && p->d != 96 && p->d != 128 && p->d != 256) return JVPATTN_ERR_HEADDIM;
  if (p->d == 256 && p->dtype == JVPATTN_F32) return JVPATTN_ERR_HEADDIM;   // 16-bit types only
  // One head of q/k (plus a partial tile of slack) must be addressable with 31-bit byte offsets,
  // and stay below the offset the kernels use to read zeros past a head's end (0x7ffffff0:
  // the padding columns of d = 32 and 96).
  const int64_t kHeadLimit = (int64_t(1) << 31) - 256;
  if ((int64_t(p->Nq) + 256) * p->d * es > kHeadLimit || (int64_t(p->Nk) + 256) * p->d * es > kHeadLimit)
    return JVPATTN_ERR_SHAPE;
  if (!std::isfinite(p->scale) || !(p->scale > 0.0f)) return JVPATTN_ERR_SCALE;

  if (p->mask_kind != JVPATTN_MASK_NONE && p->mask_kind != JVPATTN_MASK_BOOL &&
      p->mask_kind != JVPATTN_MASK_ADDITIVE && p->mask_kind != JVPATTN_MASK_BITS)
    return JVPATTN_ERR_MASK;
  const bool has_mask = p->mask_kind != JVPATTN_MASK_NONE;
  const bool work = rows_q > 0;
  int64_t mask_bytes = 0;
  int mask_es = 0;
  if (has_mask) {
    if (work && !mask) return JVPATTN_ERR_MASK;
    if (p->mask_stride_b < 0 || p->mask_stride_h < 0 || p->mask_stride_q < 0) return JVPATTN_ERR_MASK;
    mask_es = p->mask_kind == JVPATTN_MASK_BOOL ? 1 : p->mask_kind == JVPATTN_MASK_BITS ? 4 : es;
    // elements of one mask row: keys, or 32-bit words of 32 keys
    const int64_t row = p->mask_kind == JVPATTN_MASK_BITS ? (int64_t(p->Nk) + 31) / 32 : p->Nk;
    // extent = largest element offset + 1
    int64_t eb, eh, eq, ext = 0;
    if (work && p->Nk > 0) {
      if (!mul_ok(p->B - 1, p->mask_stride_b, &eb) || !mul_ok(p->H - 1, p->mask_stride_h, &eh) ||
          !mul_ok(p->Nq - 1, p->mask_stride_q, &eq))
        return JVPATTN_ERR_MASK;
      ext = eb;
      if (ext > INT64_MAX - eh) return JVPATTN_ERR_MASK;
      ext += eh;
      if (ext > INT64_MAX - eq) return JVPATTN_ERR_MASK;
      ext += eq;
      if (ext > INT64_MAX - row) return JVPATTN_ERR_MASK;
      ext += row;
      if (!mul_ok(ext, mask_es, &mask_bytes)) return JVPATTN_ERR_MASK;
      // one head's slice (rows past Nq included) must be addressable with 31-bit byte offsets
      int64_t head_rows;
      if (!mul_ok(int64_t(p->Nq) + 128, p->mask_stride_q, &head_rows) ||
          head_rows > (kHeadLimit / mask_es) - row - 64)
        return JVPATTN_ERR_MASK;
    }
  } else if (mask) {
    return JVPATTN_ERR_MASK;
  }

  if (work) {
    if (!q || !o || !to || !lse) return JVPATTN_ERR_NULL;
    if (rows_k > 0 && (!k || !v)) return JVPATTN_ERR_NULL;
  }

  const void* tensors[] = {q, k, v, tq, tk, tv, o, to};
  for (const void* t : tensors)
    if (t && !aligned(t, 16)) return JVPATTN_ERR_ALIGN;
  if ((lse && !aligned(lse, 4)) || (tlse && !aligned(tlse, 4))) return JVPATTN_ERR_ALIGN;
  if (mask && !aligned(mask, mask_es > 0 ? mask_es : 1)) return JVPATTN_ERR_ALIGN;

  if (work) {
    const Span outs[] = {span(o, bytes_q), span(to, bytes_q), span(lse, bytes_stats),
                         span(tlse, tlse ? bytes_stats : 0)};
    const Span ins[] = {span(q, bytes_q),  span(k, bytes_k),  span(v, bytes_k), span(tq, bytes_q),
                        span(tk, bytes_k), span(tv, bytes_k), span(mask, mask_bytes)};
    for (int i = 0; i < 4; ++i) {
      for (const Span& s : ins)
        if (overlap(outs[i], s)) return JVPATTN_ERR_ALIAS;
      for (int j = i + 1; j < 4; ++j)
        if (overlap(outs[i], outs[j])) return JVPATTN_ERR_ALIAS;
    }
  }

  if (sizes) {
    sizes->rows_q = rows_q;
    sizes->rows_k = rows_k;
    sizes->elem_bytes = es;
    sizes->hkv = hkv;
    sizes->group = hkv > 0 ? p->H / hkv : 1;
  }
  return JVPATTN_OK;
}

int check_fwd_tmask(const jvpattn_params* p, const void* q, const void* k, const void* v,
                    const void* tq, const void* tk, const void* tv, const void* mask, const void* tmask,
                    const void* o, const void* to, const float* lse, const float* tlse, FwdSizes* sizes) {
  FwdSizes sz;
  const int rc = check_fwd(p, q, k, v, tq, tk, tv, mask, o, to, lse, tlse, &sz);
  if (rc != JVPATTN_OK) return rc;
  if (tmask) {
    if (p->mask_kind != JVPATTN_MASK_ADDITIVE) return JVPATTN_ERR_MASK;
    if (!aligned(tmask, sz.elem_bytes)) return JVPATTN_ERR_ALIGN;
    if (sz.rows_q > 0 && p->Nk > 0) {
      // laid out as the mask: check_fwd proved this extent fits
      const int64_t bytes = ((p->B - 1) * p->mask_stride_b + (p->H - 1) * p->mask_stride_h +
                             (p->Nq - 1) * p->mask_stride_q + p->Nk) * sz.elem_bytes;
      const int64_t stats = sz.rows_q * 4, outb = sz.rows_q * p->d * sz.elem_bytes;
      const Span t = span(tmask, bytes);
      const Span outs[] = {span(o, outb), span(to, outb), span(lse, stats), span(tlse, tlse ? stats : 0)};
      for (const Span& x : outs)
        if (overlap(t, x)) return JVPATTN_ERR_ALIAS;
    }
  }
  if (sizes) *sizes = sz;
  return JVPATTN_OK;
}

thread_local int g_last_hip_error = 0;

int64_t bwd_workspace_bytes(int64_t rows_q) {
  // four float32 arrays of rows_q entries, each starting on a 256-byte boundary
  const int64_t per = (rows_q * 4 + 255) / 256 * 256;
  return 4 * per;
}

int check_bwd(const jvpattn_params* p, const void* q, const void* k, const void* v,
              const void* tq, const void* tk, const void* tv, const void* mask,
              const void* o, const void* to, const float* lse, const float* tlse,
              const void* go, const void* gto, const void* dq, const void* dk, const void* dv,
              const void* dtq, const void* dtk, const void* dtv, const void* workspace,
              size_t workspace_bytes, FwdSizes* sizes) {
  FwdSizes sz;
  // The arguments shared with the forward, checked as the forward checks them
  // (o, to, lse, tlse in the role of its outputs: present, aligned, disjoint
  // from q..mask).
  int rc = check_fwd(p, q, k, v, tq, tk, tv, mask, o, to, lse, tlse, &sz);
  if (rc != JVPATTN_OK) return rc;
  // float16 / bfloat16 with d = 64 or 128, float32 with d = 64
  if (p->dtype != JVPATTN_F16 && p->dtype != JVPATTN_BF16 && p->dtype != JVPATTN_F32) return JVPATTN_ERR_DTYPE;
  if (p->d != 64 && (p->d != 128 || p->dtype == JVPATTN_F32)) return JVPATTN_ERR_HEADDIM;
  const bool rows = sz.rows_q > 0, keys = sz.rows_k > 0;
  // go, gto may be NULL (zero cotangent); dtq, dtk, dtv may be NULL (not written)
  if (rows && (!tlse || !dq)) return JVPATTN_ERR_NULL;
  if (keys && (!dk || !dv)) return JVPATTN_ERR_NULL;
  const void* vecs[] = {go, gto, dq, dk, dv, dtq, dtk, dtv};
  for (const void* t : vecs)
    if (t && !aligned(t, 16)) return JVPATTN_ERR_ALIGN;
  const int64_t need = bwd_workspace_bytes(sz.rows_q);
  if (rows) {
    if (!workspace || static_cast<int64_t>(workspace_bytes) < need || !aligned(workspace, 256))
      return JVPATTN_ERR_WORKSPACE;
  }
  const int64_t bq = sz.rows_q * p->d * sz.elem_bytes, bk = sz.rows_k * p->d * sz.elem_bytes;
  int64_t mask_bytes = 0;
  if (mask && rows && keys) {
    const bool bits = p->mask_kind == JVPATTN_MASK_BITS;
    const int mes = p->mask_kind == JVPATTN_MASK_BOOL ? 1 : bits ? 4 : sz.elem_bytes;
    const int64_t row = bits ? (int64_t(p->Nk) + 31) / 32 : p->Nk;
    mask_bytes = ((p->B - 1) * p->mask_stride_b + (p->H - 1) * p->mask_stride_h +
                  (p->Nq - 1) * p->mask_stride_q + row) * mes;   // check_fwd proved this fits
  }
  const Span ins[] = {span(q, bq),  span(k, bk),   span(v, bk),   span(tq, bq),    span(tk, bk),
                      span(tv, bk), span(mask, mask_bytes), span(o, bq), span(to, bq),
                      span(lse, sz.rows_q * 4), span(tlse, sz.rows_q * 4), span(go, bq), span(gto, bq)};
  const Span outs[] = {span(dq, rows ? bq : 0),  span(dk, keys ? bk : 0),  span(dv, keys ? bk : 0),
                       span(dtq, rows ? bq : 0), span(dtk, keys ? bk : 0), span(dtv, keys ? bk : 0)};
  const Span ws = span(rows ? workspace : nullptr, rows ? need : 0);
  for (int i = 0; i < 6; ++i) {
    for (const Span& in : ins)
      if (overlap(outs[i], in)) return JVPATTN_ERR_ALIAS;
    for (int j = i + 1; j < 6; ++j)
      if (overlap(outs[i], outs[j])) return JVPATTN_ERR_ALIAS;
    if (overlap(outs[i], ws)) return JVPATTN_ERR_WORKSPACE;
  }
  for (const Span& in : ins)
    if (overlap(ws, in)) return JVPATTN_ERR_WORKSPACE;
  if (sizes) *sizes = sz;
  return JVPATTN_OK;
}

int check_bwd_tmask(const jvpattn_params* p, const void* q, const void* k, const void* v,
                    const void* tq, const void* tk, const void* tv, const void* mask, const void* tmask,
                    const void* o, const void* to, const float* lse, const float* tlse,
                    const void* go, const void* gto, const void* dq, const void* dk, const void* dv,
                    const void* dtq, const void* dtk, const void* dtv, const void* workspace,
                    size_t workspace_bytes, FwdSizes* sizes) {
  FwdSizes sz;
  int rc = check_bwd(p, q, k, v, tq, tk, tv, mask, o, to, lse, tlse, go, gto, dq, dk, dv, dtq, dtk, dtv,
                     workspace, workspace_bytes, &sz);
  if (rc != JVPATTN_OK) return rc;
  // the forward's rules for tmask (o, to, lse, tlse as the spans it must avoid) ...
  rc = check_fwd_tmask(p, q, k, v, tq, tk, tv, mask, tmask, o, to, lse, tlse, nullptr);
  if (rc != JVPATTN_OK) return rc;
  // ... and none of the reverse pass's outputs or workspace may overlap it
  if (tmask && sz.rows_q > 0 && p->Nk > 0) {
    const int64_t bytes = ((p->B - 1) * p->mask_stride_b + (p->H - 1) * p->mask_stride_h +
                           (p->Nq - 1) * p->mask_stride_q + p->Nk) * sz.elem_bytes;
    const int64_t bq = sz.rows_q * p->d * sz.elem_bytes, bk = sz.rows_k * p->d * sz.elem_bytes;
    const Span t = span(tmask, bytes);
    const Span outs[] = {span(dq, bq), span(dk, bk), span(dv, bk), span(dtq, bq), span(dtk, bk), span(dtv, bk)};
    for (const Span& x : outs)
      if (overlap(t, x)) return JVPATTN_ERR_ALIAS;
    if (overlap(t, span(workspace, bwd_workspace_bytes(sz.rows_q)))) return JVPATTN_ERR_WORKSPACE;
  }
  if (sizes) *sizes = sz;
  return JVPATTN_OK;
}

}  // namespace jvpattn

extern "C" int jvpattn_check_bwd_tmask(const jvpattn_params* params, const void* q, const void* k,
                                       const void* v, const void* tq, const void* tk, const void* tv,
                                       const void* mask, const void* tmask, const void* o, const void* to,
                                       const float* lse, const float* tlse, const void* go, const void* gto,
                                       const void* dq, const void* dk, const void* dv, const void* dtq,
                                       const void* dtk, const void* dtv, const void* workspace,
                                       size_t workspace_bytes) {
  return jvpattn::check_bwd_tmask(params, q, k, v, tq, tk, tv, mask, tmask, o, to, lse, tlse, go, gto, dq, dk,
                                  dv, dtq, dtk, dtv, workspace, workspace_bytes, nullptr);
}

extern "C" int jvpattn_last_hip_error(void) { return jvpattn::g_last_hip_error; }

extern "C" int64_t jvpattn_bwd_workspace_bytes(const jvpattn_params* p) {
  if (!p) return JVPATTN_ERR_NULL;
  if (p->B < 0 || p->H < 0 || p->Nq < 0) return JVPATTN_ERR_SHAPE;
  int64_t bh = int64_t(p->B) * p->H;
  if (p->Nq > 0 && bh > INT64_MAX / 4 / p->Nq) return JVPATTN_ERR_SHAPE;
  return jvpattn::bwd_workspace_bytes(bh * p->Nq);
}

extern "C" int jvpattn_check_bwd(const jvpattn_params* params, const void* q, const void* k,
                                 const void* v, const void* tq, const void* tk, const void* tv,
                                 const void* mask, const void* o, const void* to, const float* lse,
                                 const float* tlse, const void* go, const void* gto, const void* dq,
                                 const void* dk, const void* dv, const void* dtq, const void* dtk,
                                 const void* dtv, const void* workspace, size_t workspace_bytes) {
  return jvpattn::check_bwd(params, q, k, v, tq, tk, tv, mask, o, to, lse, tlse, go, gto, dq, dk, dv,
                            dtq, dtk, dtv, workspace, workspace_bytes, nullptr);
}

extern "C" int jvpattn_check_fwd_tmask(const jvpattn_params* params, const void* q, const void* k,
                                       const void* v, const void* tq, const void* tk, const void* tv,
                                       const void* mask, const void* tmask, const void* o, const void* to,
                                       const float* lse, const float* tlse) {
  return jvpattn::check_fwd_tmask(params, q, k, v, tq, tk, tv, mask, tmask, o, to, lse, tlse, nullptr);
}

extern "C" int jvpattn_check_fwd(const jvpattn_params* params, const void* q, const void* k,
                                 const void* v, const void* tq, const void* tk, const void* tv,
                                 const void* mask, const void* o, const void* to, const float* lse,
                                 const float* tlse) {
  return jvpattn::check_fwd(params, q, k, v, tq, tk, tv, mask, o, to, lse, tlse, nullptr);
}

extern "C" const char* jvpattn_strerror(int code) {
  switch (code) {
    case JVPATTN_OK: return "ok";
    case JVPATTN_ERR_NULL: return "a required pointer is NULL";
    case JVPATTN_ERR_SHAPE:
      return "invalid shape (negative size, d <= 0, Hkv not a divisor of H, or size overflow)";
    case JVPATTN_ERR_DTYPE: return "unknown dtype";
    case JVPATTN_ERR_HEADDIM: return "unsupported head dimension (forward: 32, 64, 96, 128, and 256 for 16-bit types; reverse pass: 64)";
    case JVPATTN_ERR_MASK: return "invalid mask (unknown kind, pointer/kind mismatch, or bad strides)";
    case JVPATTN_ERR_ALIGN: return "misaligned pointer (tensors: 16 bytes, lse/tlse: 4 bytes)";
    case JVPATTN_ERR_SCALE: return "scale must be finite and > 0";
    case JVPATTN_ERR_ALIAS: return "an output overlaps an input or another output";
    case JVPATTN_ERR_HIP: return "HIP runtime error on launch";
    case JVPATTN_ERR_WORKSPACE: return "workspace missing, too small, not 256-byte aligned, or overlapping";
    case JVPATTN_ERR_ARG: return "argument outside its documented range";
    case JVPATTN_ERR_SCRATCH: return "B*H*Nq exceeds the fixed scratch of jvpattn_bwd_noalloc (2^20 rows)";
    default: return "unknown error code";
  }
}
