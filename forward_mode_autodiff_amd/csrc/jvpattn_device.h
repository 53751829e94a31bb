// Device helpers shared by the forward and reverse kernels for gfx950:
// vector types, the 16-bit element types, buffer resources, the LDS tile
// layout and transpose reads, waits and barriers, masks, and the
// online-softmax steps of the 16-bit kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "jvpattn.h"
#include "jvpattn_fwd_launch.h"

namespace jvpattn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kTileThreads = 256;     // threads that fill one LDS tile (4 waves)


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));


// Maximum of three values. IEEE maximum (NaN-propagating) fuses into one
// v_maximum3_f32 with no NaN canonicalisation of matrix-core results, which a
// chain of fmaxf would need. Written as a builtin, not asm, so the compiler
// sees the read of matrix-core destinations and inserts the wait states
// gfx950 requires before a vector instruction may read them (it does not look
// inside inline asm: an asm reader could see a partial accumulation).
__device__ inline float max3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// ---------------------------------------------------------------- 16-bit types

struct BF16 {
  using vec8 = bf16x8;
  static constexpr uint32_t kNegInf16 = 0xff80u;   // -inf
  __device__ static inline f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack2(float a, float b) {
    f32x2 f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
  }
  __device__ static inline float widen(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }
  // x times a power of two s, rounded back (exact: bfloat16 has float32's exponent range)
  __device__ static inline vec8 scale8(vec8 x, float s) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = static_cast<__bf16>(static_cast<float>(x[e]) * s);
    return x;
  }
  // acc + the two 16-bit values of w
  __device__ static inline float dot2sum(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, 0x3f803f80u),
                                           acc, false);
  }
  // Weights must be rebased when a lane's 16 weights sum past 2^12 (so each is
  // at most 2^12; bfloat16 and the float32 sums have range to spare).
  __device__ static inline bool spill(float lane_sum, const float (&)[16]) { return !(lane_sum <= 4096.0f); }
};

struct F16 {
  using vec8 = f16x8;
  static constexpr uint32_t kNegInf16 = 0xfc00u;   // -inf
  __device__ static inline f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack2(float a, float b) {
    f32x2 f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
  }
  __device__ static inline float widen(uint16_t x) {
    return static_cast<float>(__builtin_bit_cast(_Float16, x));
  }
  // x times a power of two s, rounded back: exact unless the product falls below
  // float16's normal range (2^-14), where it rounds to the subnormal grid (error <= 2^-25)
  __device__ static inline vec8 scale8(vec8 x, float s) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = static_cast<_Float16>(static_cast<float>(x[e]) * s);
    return x;
  }
  __device__ static inline float dot2sum(uint32_t w, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), __builtin_bit_cast(f16x2, 0x3c003c00u), acc, false);
  }
  // Weights must be rebased when a lane's 16 weights sum past 2^6, so each
  // is at most 2^6 (products with score tangents past float16's range are
  // caught by f16_range_guard).
  __device__ static inline bool spill(float lane_sum, const float (&)[16]) { return !(lane_sum <= 64.0f); }
};

__device__ inline uint32_t lo16(uint32_t x) { return x & 0xffffu; }
__device__ inline uint32_t hi16(uint32_t x) { return x >> 16; }

// A buffer offset past every record (one head is at most 2 GiB - 256 rows): loads read zeros,
// stores are dropped.
constexpr int kOutOfRange = 0x7ffffff0;

// Buffer resources: loads at byte offsets >= the record count return zero, so
// ragged tails and absent (NULL) tangents need no branches.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;

__device__ inline Rsrc make_rsrc(const void* p, int64_t bytes) {
  const int64_t n = bytes <= 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(n), kRsrcWord3);
}
__device__ inline uint4 ld128(Rsrc r, int off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ inline uint2 ld64(Rsrc r, int off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

// Values of lanes l and l^32 combined (both halves receive the result).
__device__ inline float xhalf_max(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ inline float xhalf_sum(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

template <typename V, typename P>
__device__ inline V lds_load(const P* base, int off) {
  return *reinterpret_cast<const V*>(reinterpret_cast<const char*>(base) + off);
}
template <typename V, typename P>
__device__ inline void lds_store(P* base, int off, V x) {
  *reinterpret_cast<V*>(reinterpret_cast<char*>(base) + off) = x;
}

template <int D>
struct Tile16 {
  static constexpr int BN = 32;                   // keys per LDS tile (one 32-key block)
  static constexpr int NC = D / 16;               // 16-wide chunks of the head dimension
  static constexpr int NT = D / 32;               // 32-row tiles of the output
  static constexpr int GR = D / 8;                // 16-byte granules per row
  static constexpr int ROW = 2 * D;               // bytes per row
  static constexpr int TENSOR_BYTES = BN * ROW;
  static constexpr int STAGE_BYTES = 4 * TENSOR_BYTES;          // K, dK, V, dV
  static constexpr int LOADS = TENSOR_BYTES / (16 * kTileThreads);  // 16-byte loads per thread per tensor
  static constexpr int TILE_VMEM = 4 * LOADS;                   // direct loads per thread per tile
  static_assert(LOADS * 16 * kTileThreads == TENSOR_BYTES, "tile must split evenly over the workgroup");
};

// Bytes per mask element: uint8 for bool, 32-bit words for bit-packed masks,
// else the additive values (value_bytes).
template <int MASK>
constexpr int mask_es(int value_bytes) {
  return MASK == JVPATTN_MASK_BOOL ? 1 : MASK == JVPATTN_MASK_BITS ? 4 : value_bytes;
}

// float32 tiles of 32 rows (keys, or queries in the reverse pass): rows as
// 16-byte granules XOR-swizzled by row (the A operands of the score-like
// products), and transposed tiles whose row is a head-dim index holding the
// 32 rows' values, 4 per granule (the A operands of the accumulating products).
template <int D>
struct Tile32 {
  static constexpr int BN = 32;                 // rows per LDS tile
  static constexpr int NT = D / 32;
  static constexpr int GR = D / 4;              // 16-byte granules per row
  static constexpr int TENSOR_BYTES = BN * D * 4;
  static constexpr int BUF_BYTES = 4 * TENSOR_BYTES;
};

template <int D>
__device__ inline int k32_off(int row, int g) {
  return row * (4 * D) + ((g ^ (row & 7)) << 4);
}
// transposed tile: row = head-dim index, 32 values (128 bytes, 8 granules)
__device__ inline int vt32_off(int dd, int g) { return dd * 128 + ((g ^ (dd & 7)) << 4); }

// LDS tiles (K, dK, V, dV) are row = key, 2*D bytes per row, with the 16-byte
// granules of a row XOR-swizzled by swz(row). They are filled by direct
// global->LDS loads: load slot p (16 bytes) of a tile lands at byte 16*p,
// i.e. at (row, physical granule) = (p / GR, p % GR), so the lane that owns
// slot p fetches logical granule (p % GR) ^ swz(row) of that row.
#ifndef JVPATTN_SWZ
#define JVPATTN_SWZ 1
#endif
__device__ inline int swz(int row) {
#if JVPATTN_SWZ == 0
  return row & 7;
#elif JVPATTN_SWZ == 1
  // 8 consecutive rows -> 8 distinct granules (K reads), and 4 consecutive rows
  // -> 4 distinct granule pairs (transpose reads of 2 adjacent granules).
  return ((row & 3) << 1) | ((row >> 2) & 1);
#else
  return (row >> 1) & 7;
#endif
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ inline lds_char* to_lds(const char* p) { return (lds_char*)(p); }

// 4 keys x 16 head-dim columns -> each of 16 lanes gets one column: the LDS
// transpose read of gfx950. In every group of 16 lanes, lane i returns
// element (i % 4) of the 8 bytes addressed by lane 4*e + i/4, for e = 0..3.
__device__ inline v4i16 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)to_lds(p));
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (loads and stores retire in issue order on this target, so this means all
// but the N most recent have completed).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt is a 6-bit count");
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

// Buffer stores: offsets at or past the record count are dropped, so a
// wave can issue a fixed number of stores whatever its rows and columns.
__device__ inline void st64(Rsrc r, int off, uint2 v) {
  typedef unsigned int v2u __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(v2u{v.x, v.y}, r, off, 0, 0);
}
__device__ inline void st32(Rsrc r, int off, uint32_t v) { __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0); }

// Workgroup barrier for the LDS ring. The caller has already waited for its
// own direct-to-LDS loads (wait_vmcnt); this waits for its LDS reads and
// syncs. (A fenced __syncthreads would also drain every in-flight tile load.)
// Builtins rather than inline assembly, so the compiler's own wait
// insertion knows that LDS reads issued before the barrier have completed.
__device__ inline void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0); vmcnt, expcnt unconstrained
  __builtin_amdgcn_s_barrier();
}


// Mask values of one 32-key block for this lane's 16 keys, loaded ahead of use.
template <int MASK> struct MaskVals {};
template <> struct MaskVals<JVPATTN_MASK_BOOL> { uint32_t w[4]; };
template <> struct MaskVals<JVPATTN_MASK_ADDITIVE> { uint2 w[4]; };
template <> struct MaskVals<kMaskAddT> { uint2 w[4]; uint2 t[4]; };   // mask, its tangent
template <> struct MaskVals<JVPATTN_MASK_BITS> { uint32_t w; };          // the block's word >> 4*hlf

// Register r of this lane holds key k0 + 8*(r/4) + 4*hlf + r%4.
// Args: any argument block with Nk, msq (mask row stride) and mask_vec.
template <int MASK, typename Args>
__device__ inline void mask_load(MaskVals<MASK>& m, const Args& a, Rsrc mr, int qi, int k0, int hlf);

// Additive mask and its tangent (resource mtr, same element layout).
template <typename Args>
__device__ inline void mask_load_t(MaskVals<kMaskAddT>& m, const Args& a, Rsrc mr, Rsrc mtr, int qi, int k0,
                                   int hlf) {
  MaskVals<JVPATTN_MASK_ADDITIVE> x, y;
  mask_load<JVPATTN_MASK_ADDITIVE>(x, a, mr, qi, k0, hlf);
  mask_load<JVPATTN_MASK_ADDITIVE>(y, a, mtr, qi, k0, hlf);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    m.w[g] = x.w[g];
    m.t[g] = y.w[g];
  }
}

template <int MASK, typename Args>
__device__ inline void mask_load(MaskVals<MASK>& m, const Args& a, Rsrc mr, int qi, int k0, int hlf) {
  if constexpr (MASK == JVPATTN_MASK_BITS) {
    // one 32-bit word holds the block (k0 is a multiple of 32); this lane's
    // keys 4*hlf + 8g + e sit at bit 8g + e once shifted by 4*hlf
    // (a rotation rather than a shift: the bits read stay below bit 28, and the compiler keeps one
    // rotate instead of folding the lane's offset into every bit extraction)
    const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(mr, (qi * int(a.msq) + (k0 >> 5)) * 4, 0, 0);
    m.w = __builtin_amdgcn_alignbit(w, w, 4 * hlf);
  }
  if constexpr (MASK == JVPATTN_MASK_BOOL || MASK == JVPATTN_MASK_ADDITIVE) {
    constexpr int es = MASK == JVPATTN_MASK_BOOL ? 1 : 2;
    // byte offset of (qi, k0 + 4*hlf) in this head's mask; rows past Nq are never stored
    const int row = (qi * int(a.msq) + k0 + 4 * hlf) * es;
    const bool vec = a.mask_vec && k0 + 32 <= a.Nk;
    if constexpr (MASK == JVPATTN_MASK_BOOL) {
      if (vec) {
#pragma unroll
        for (int g = 0; g < 4; ++g) m.w[g] = __builtin_amdgcn_raw_buffer_load_b32(mr, row + 8 * g, 0, 0);
      } else {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          m.w[g] = 0u;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            m.w[g] |= uint32_t(__builtin_amdgcn_raw_buffer_load_b8(mr, row + 8 * g + e, 0, 0)) << (8 * e);
        }
      }
    } else {
      if (vec) {
#pragma unroll
        for (int g = 0; g < 4; ++g) m.w[g] = ld64(mr, row + 16 * g);
      } else {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint32_t e4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) e4[e] = __builtin_amdgcn_raw_buffer_load_b16(mr, row + 16 * g + 2 * e, 0, 0);
          m.w[g].x = e4[0] | (e4[1] << 16);
          m.w[g].y = e4[2] | (e4[3] << 16);
        }
      }
    }
  }
}

// Scores in score units: raw q.k without an additive mask (scale folded into
// cx), scale q.k + M with one. PRESCALED: s already holds scale q.k.
template <typename T, int MASK, bool PRESCALED>
__device__ inline void mask_apply(f32x16& s, const MaskVals<MASK>& m, float scale) {
  if constexpr (MASK == JVPATTN_MASK_BITS) {
    // the key's bit sign-extended to all ones or zero selects the score or -inf (bitfield insert)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t sel = uint32_t(__builtin_amdgcn_sbfe(int(m.w), 8 * (r >> 2) + (r & 3), 1));
      s[r] = __uint_as_float((__float_as_uint(s[r]) & sel) | (0xff800000u & ~sel));
    }
  } else if constexpr (MASK == JVPATTN_MASK_BOOL) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (((m.w[r >> 2] >> (8 * (r & 3))) & 0xffu) == 0u) s[r] = -INFINITY;
  } else if constexpr (MASK == JVPATTN_MASK_ADDITIVE || MASK == kMaskAddT) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint2 x = m.w[r >> 2];
      const uint32_t word = (r & 2) ? x.y : x.x;
      const uint16_t bits = (r & 1) ? hi16(word) : lo16(word);
      s[r] = PRESCALED ? s[r] + T::widen(bits) : fmaf(s[r], scale, T::widen(bits));
    }
  }
}

// With a mask tangent: sd (score tangent in units where sd * us = dS) gains
// dM / us; inv_us = 1 / us. No-op for the other kinds.
template <typename T, int MASK>
__device__ inline void mask_tangent(f32x16& sd, const MaskVals<MASK>& m, float inv_us) {
  if constexpr (MASK == kMaskAddT) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint2 x = m.t[r >> 2];
      const uint32_t word = (r & 2) ? x.y : x.x;
      const uint16_t bits = (r & 1) ? hi16(word) : lo16(word);
      sd[r] = fmaf(T::widen(bits), inv_us, sd[r]);
    }
  }
}

// Whether the mask values m (this lane's 16 keys of a 32-key block) leave any
// key visible: nonzero bool bytes or bits, additive values other than -inf.
// A block no lane of a wave sees (the mask hides all 32 x 32 entries) adds
// nothing to that wave's rows, so the wave skips its softmax and value
// products. Causal and ragged-tail hiding are not looked at (those blocks
// then just run).
template <typename T, int MASK>
__device__ inline bool mask_any_visible(const MaskVals<MASK>& m) {
  if constexpr (MASK == JVPATTN_MASK_BOOL) {
    return ((m.w[0] | m.w[1]) | (m.w[2] | m.w[3])) != 0u;
  } else if constexpr (MASK == JVPATTN_MASK_BITS) {
    return (m.w & 0x0f0f0f0fu) != 0u;   // this lane's keys sit at bits 8g + e, e < 4
  } else if constexpr (MASK == JVPATTN_MASK_ADDITIVE || MASK == kMaskAddT) {
    constexpr uint32_t ninf = T::kNegInf16 | (T::kNegInf16 << 16);
    uint32_t all = m.w[0].x & m.w[0].y, any = m.w[0].x | m.w[0].y;
#pragma unroll
    for (int g = 1; g < 4; ++g) {
      all &= m.w[g].x & m.w[g].y;
      any |= m.w[g].x | m.w[g].y;
    }
    return !(all == ninf && any == ninf);   // some value differs from -inf
  } else {
    return true;
  }
}

// Keys past Nk, and (causal) keys after the query, get score -inf.
template <bool CAUSAL>
__device__ inline void hide_keys(f32x16& s, int Nk, int qi, int k0, int hlf) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = k0 + (r >> 2) * 8 + 4 * hlf + (r & 3);
    bool hide = key >= Nk;
    if constexpr (CAUSAL) hide = hide || key > qi;
    if (hide) s[r] = -INFINITY;
  }
}

// Mask resource of head (b, h): element (i, j) at byte (i*msq + j) * es.
// `base` is the mask (default) or a tensor laid out like it (its tangent).
// A bit-packed mask (es = 4 with bits) has ceil(Nk/32) words per row.
template <typename Args>
__device__ inline Rsrc mask_rsrc(const Args& a, int b, int h, int es, const void* base = nullptr,
                                 bool bits = false) {
  const void* m = base ? base : a.mask;
  if (!m) return make_rsrc(a.q, 0);
  const int64_t off = (b * a.msb + h * a.msh) * es;
  const int64_t row = bits ? (a.Nk + 31) >> 5 : a.Nk;
  const int64_t bytes = (int64_t(a.Nq - 1) * a.msq + row) * es;
  return make_rsrc(static_cast<const char*>(m) + off, bytes);
}

// Largest score of this lane's query column (both lane halves).
__device__ inline float block_max(const f32x16& s) {
  float m = max3(s[0], s[1], s[2]);
#pragma unroll
  for (int r = 3; r < 15; r += 2) m = max3(m, s[r], s[r + 1]);
  m = max3(m, s[15], s[15]);
  const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return max3(__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[1]));
}

// Sum of 16 values as a balanced tree (independent adds, depth 4).
__device__ inline float sum16(const float (&x)[16]) {
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = x[2 * i] + x[2 * i + 1];
  const float b0 = a[0] + a[1], b1 = a[2] + a[3], b2 = a[4] + a[5], b3 = a[6] + a[7];
  return (b0 + b1) + (b2 + b3);
}

// Online softmax of one 32-key block for the 16-bit kernels, without a row
// maximum in the common case. The weights are first taken against the
// current reference, e = 2^(s cx - moff). A reference only has to keep the
// weights bounded (every accumulator is rescaled with it), so the block is
// accepted when this lane's 16 weights sum to at most T::kSpill, which bounds
// each of them. Otherwise -- or while the row has seen no visible key -- the
// whole wave takes the rare path: exact block maximum over both lane halves,
// raise the reference to it, rescale l and mu (alpha returned for the
// accumulators), recompute the weights. A reference set this way is always a
// score of the row, so weights of later keys far below it may underflow to 0
// only where they are negligible against that key's weight of 1.
//
// s holds the scores on entry (score units) and is clobbered; sd the score
// tangents (times us gives dS). Outputs: pB = e, uB = e dS as 16-bit B
// operands for keys 16kc .. 16kc+15.
struct RowState16 {
  float moff;    // reference in log2 units; 0 until a visible key is seen
  float l;       // this lane's partial sum of weights
  float mu;      // this lane's partial sum of weights * dS
  bool seen;     // some visible key has set the reference
};

// Step 1: weights e of the block (s is clobbered), l updated; returns true
// (and alpha for the accumulators) when the reference moved.
template <typename T>
__device__ inline bool block_exp16(f32x16& s, RowState16& st, float cx, float (&e)[16], float& alpha,
                                   float& lane_sum) {
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = fmaf(s[r], cx, -st.moff);
#pragma unroll
  for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(s[r]);
  float lt = sum16(e);
  alpha = 1.0f;
  const bool moved = __any(T::spill(lt, e) || !st.seen);
  if (moved) {
    const float bx = block_max(s);   // max over the query column of s cx - moff
    // Raise the reference only (alpha <= 1); an unseen row takes the block's
    // maximum as it is (up or down), unless every key so far is hidden (bx = -inf).
    const float shift = st.seen ? fmaxf(bx, 0.0f) : (bx > -INFINITY ? bx : 0.0f);
    // An unseen row has accumulated nothing (all zeros); its shift may be far
    // below 0, where exp2(-shift) would overflow and turn those zeros into NaN.
    alpha = st.seen ? __builtin_amdgcn_exp2f(-shift) : 0.0f;
    st.seen = st.seen || bx > -INFINITY;
    st.moff += shift;
    st.l *= alpha;
    st.mu *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(s[r] - shift);
    lt = sum16(e);
  }
  st.l += lt;
  lane_sum = lt;
  return moved;
}

// Largest magnitude of 16 values (NaN-propagating).
__device__ inline float absmax16(const float (&x)[16]) {
  float m = max3(__builtin_fabsf(x[0]), __builtin_fabsf(x[1]), __builtin_fabsf(x[2]));
#pragma unroll
  for (int r = 3; r < 15; r += 2) m = max3(m, __builtin_fabsf(x[r]), __builtin_fabsf(x[r + 1]));
  return __builtin_elementwise_maximum(m, __builtin_fabsf(x[15]));
}

// float16 range guard. A weight times its score tangent, rounded to float16,
// overflows past 65504: with weights kept up to 2^6 (2^4 in the 4-wave
// kernel) against the running reference, once |dS| reaches 2^10 (2^12).
// lane_sum * max |dS| over the lane's 16 keys bounds every such product; when
// a query column's bound (both lane halves) reaches 2^15, its reference rises
// by the smallest k that brings the bound under 2^14: its weights, l (which
// already holds this block's weights) and mu (which does not) shrink by 2^-k,
// moff grows by k, and the returned factor 2^-k (1 for every other column)
// tells the caller to shrink the column's accumulators, which do not hold this
// block yet. ds_scale turns sd into dS. A non-finite bound (a non-finite
// input) moves nothing. The check is uniform over the wave; the rescale is
// taken only when some column needs it.
template <typename E>
__device__ inline float f16_range_guard(E& e, const f32x16& sd, float ds_scale, float lane_sum, float& moff,
                                        float& l, float& mu) {
  float a[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) a[r] = sd[r];
  const float bound = lane_sum * (absmax16(a) * ds_scale);
  if (!__any(!(bound < 32768.0f))) return 1.0f;
  const float need = xhalf_max(bound);
  const float k = (need >= 32768.0f && need <= 3.0e38f) ? ceilf(__builtin_amdgcn_logf(need)) - 14.0f : 0.0f;
  const float f = __builtin_amdgcn_exp2f(-k);
#pragma unroll
  for (int r = 0; r < 16; ++r) e[r] *= f;
  moff += k;
  l *= f;
  mu *= f;
  return f;
}

// Step 2: pB = e and uB = e dS (dS = sd, times us when SCALED_U) as 16-bit B
// operands for keys 16kc .. 16kc+15. E: any 16-element float container.
template <typename T, bool SCALED_U, typename E>
__device__ inline void block_pack16(const E& e, const f32x16& sd, float us, typename T::vec8 (&pB)[2],
                                    typename T::vec8 (&uB)[2]) {
  uint32_t pw[8], uw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    pw[i] = T::pack2(e[2 * i], e[2 * i + 1]);
    const float u0 = SCALED_U ? (sd[2 * i] * us) * e[2 * i] : sd[2 * i] * e[2 * i];
    const float u1 = SCALED_U ? (sd[2 * i + 1] * us) * e[2 * i + 1] : sd[2 * i + 1] * e[2 * i + 1];
    uw[i] = T::pack2(u0, u1);
  }
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    pB[kc] = __builtin_bit_cast(typename T::vec8, uint4{pw[4 * kc], pw[4 * kc + 1], pw[4 * kc + 2], pw[4 * kc + 3]});
    uB[kc] = __builtin_bit_cast(typename T::vec8, uint4{uw[4 * kc], uw[4 * kc + 1], uw[4 * kc + 2], uw[4 * kc + 3]});
  }
}

// Sum of the 16 rounded products held in uB (the values the value products use).
template <typename T>
__device__ inline float block_mu_part(const typename T::vec8 (&uB)[2]) {
  const uint4 a = __builtin_bit_cast(uint4, uB[0]), b = __builtin_bit_cast(uint4, uB[1]);
  float m0 = T::dot2sum(a.x, 0.0f), m1 = T::dot2sum(b.x, 0.0f);
  m0 = T::dot2sum(a.y, m0);
  m1 = T::dot2sum(b.y, m1);
  m0 = T::dot2sum(a.z, m0);
  m1 = T::dot2sum(b.z, m1);
  m0 = T::dot2sum(a.w, m0);
  m1 = T::dot2sum(b.w, m1);
  return m0 + m1;
}

// mu += the 16 rounded products held in uB.
template <typename T>
__device__ inline void block_mu16(const typename T::vec8 (&uB)[2], RowState16& st) {
  st.mu += block_mu_part<T>(uB);
}

}  // namespace
}  // namespace jvpattn
