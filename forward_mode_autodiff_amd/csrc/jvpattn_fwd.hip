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
// V and dV are stored transposed in LDS (with the key order permuted to
// match the C layout) so that V^T A-operands are single 16-byte LDS reads.
// The score tangent uses one chain over 2d: dS^T = dK Q^T + K dQ^T.
// The two tangent products share one accumulator: accT += V^T (P dS)^T + dV^T P^T.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "jvpattn.h"
#include "jvpattn_internal.h"

namespace jvpattn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWaves = 4;             // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;      // query rows per workgroup

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* tq;
  const void* tk;
  const void* tv;
  const void* mask;
  void* o;
  void* to;
  float* lse;
  float* tlse;
  int H, Nq, Nk, BH;
  int n_qblk;
  int mask_vec;       // 1: mask rows may be read 4 keys at a time
  int64_t msb, msh, msq;
  float scale;
  float cx;           // score units -> log2 units
  float thr;          // lazy-rescale threshold in score units
};

// ---------------------------------------------------------------- 16-bit types

struct BF16 {
  using vec8 = bf16x8;
  static constexpr float kTau = 8.0f;   // weights may grow to 2^8 before a rescale
  __device__ static inline f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack2(float a, float b) {
    f32x2 f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
  }
  __device__ static inline float widen(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }
};

struct F16 {
  using vec8 = f16x8;
  // float16 weights times score tangents must stay below 65504: keep weights <= 2^4.
  static constexpr float kTau = 4.0f;
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
};

template <int D>
struct Tile16 {
  static constexpr int BN = D == 64 ? 64 : 32;    // keys per LDS tile
  static constexpr int KB = BN / 32;              // 32-key blocks per tile
  static constexpr int NC = D / 16;               // 16-wide chunks of the head dimension
  static constexpr int NT = D / 32;               // 32-row tiles of the output
  static constexpr int GR = D / 8;                // 16-byte granules per K row
  static constexpr int VG = BN / 8;               // 16-byte granules per V^T row
  static constexpr int TENSOR_BYTES = BN * D * 2;
  static constexpr int BUF_BYTES = 4 * TENSOR_BYTES;  // K, dK, V^T, dV^T
  static_assert(BN * GR == 2 * kThreads, "K tile = two 16-byte granules per thread");
  static_assert((BN / 4) * (D / 4) == kThreads, "V tile = one 4x4 block per thread");
};

// K / dK tile in LDS: row = key, 2*D bytes per row, 16-byte granules XOR-swizzled by row.
template <int D>
__device__ inline int k_off(int row, int g) {
  return row * (2 * D) + ((g ^ (row & 7)) << 4);
}

// V^T / dV^T tile in LDS: row = head-dimension index, 2*BN bytes per row.
template <int D>
__device__ inline int vt_swz(int dd) {
  return (dd ^ (dd >> 2)) & (Tile16<D>::VG - 1);
}
template <int D>
__device__ inline int vt_off(int dd, int g) {
  return dd * (2 * Tile16<D>::BN) + ((g ^ vt_swz<D>(dd)) << 4);
}

// Key order inside each 16-key chunk of a V^T row: bits 2 and 3 of the key
// index swapped, so that the 8 keys lane half h holds in C registers 0..7
// (keys 4h..4h+3 and 8+4h..8+4h+3) sit in 16 contiguous bytes.
__device__ inline int key_pos(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

__device__ inline uint32_t lo16(uint32_t x) { return x & 0xffffu; }
__device__ inline uint32_t hi16(uint32_t x) { return x >> 16; }

// Column c (0..3) of a 4x4 block of 16-bit values held as 4 rows of uint2.
__device__ inline uint32_t col_pair(uint2 a, uint2 b, int c) {
  uint32_t ea = c == 0 ? lo16(a.x) : c == 1 ? hi16(a.x) : c == 2 ? lo16(a.y) : hi16(a.y);
  uint32_t eb = c == 0 ? lo16(b.x) : c == 1 ? hi16(b.x) : c == 2 ? lo16(b.y) : hi16(b.y);
  return ea | (eb << 16);
}

template <typename V, typename P>
__device__ inline V lds_load(const P* base, int off) {
  return *reinterpret_cast<const V*>(reinterpret_cast<const char*>(base) + off);
}
template <typename V, typename P>
__device__ inline void lds_store(P* base, int off, V x) {
  *reinterpret_cast<V*>(reinterpret_cast<char*>(base) + off) = x;
}

// Per-row softmax state for one lane (both lanes of a query column hold the same m).
struct RowState {
  float m;       // reference maximum in score units (-inf until a visible key is seen)
  float moff;    // m * cx, or 0 while m is -inf
  float l;       // partial sum of weights over this lane's keys
  float mu;      // partial sum of weights * raw score tangent
};

// Score of register r of this lane after masking, in score units:
// MASK_NONE/BOOL: raw q.k (scale folded into cx); ADDITIVE: scale q.k + M.
template <typename T, int MASK, bool CAUSAL>
__device__ inline void mask_scores(f32x16& s, const FwdArgs& a, int b, int h, int qi, int k0, int hlf,
                                   bool elem_mask) {
  if constexpr (MASK == JVPATTN_MASK_BOOL || MASK == JVPATTN_MASK_ADDITIVE) {
    const bool row_ok = qi < a.Nq;
    const int64_t row = b * a.msb + h * a.msh + int64_t(qi) * a.msq;
    if constexpr (MASK == JVPATTN_MASK_BOOL) {
      const uint8_t* mp = static_cast<const uint8_t*>(a.mask) + row;
      uint32_t w[4] = {0u, 0u, 0u, 0u};
      if (row_ok) {
        if (a.mask_vec && k0 + 32 <= a.Nk) {
#pragma unroll
          for (int g = 0; g < 4; ++g) w[g] = *reinterpret_cast<const uint32_t*>(mp + k0 + 8 * g + 4 * hlf);
        } else {
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int key = k0 + 8 * g + 4 * hlf + e;
              if (key < a.Nk) w[g] |= uint32_t(mp[key] != 0) << (8 * e);
            }
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (((w[r >> 2] >> (8 * (r & 3))) & 0xffu) == 0u) s[r] = -INFINITY;
    } else {
      const uint16_t* mp = static_cast<const uint16_t*>(a.mask) + row;
      uint2 w[4] = {};
      if (row_ok) {
        if (a.mask_vec && k0 + 32 <= a.Nk) {
#pragma unroll
          for (int g = 0; g < 4; ++g) w[g] = *reinterpret_cast<const uint2*>(mp + k0 + 8 * g + 4 * hlf);
        } else {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            uint32_t e4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int key = k0 + 8 * g + 4 * hlf + e;
              e4[e] = key < a.Nk ? mp[key] : 0u;
            }
            w[g].x = e4[0] | (e4[1] << 16);
            w[g].y = e4[2] | (e4[3] << 16);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint2 x = w[r >> 2];
        const uint32_t word = (r & 2) ? x.y : x.x;
        const uint16_t bits = (r & 1) ? hi16(word) : lo16(word);
        s[r] = fmaf(s[r], a.scale, T::widen(bits));
      }
    }
  }
  if (elem_mask) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + (r >> 2) * 8 + 4 * hlf + (r & 3);
      bool hide = key >= a.Nk;
      if constexpr (CAUSAL) hide = hide || key > qi;
      if (hide) s[r] = -INFINITY;
    }
  }
}

// Online-softmax update for one 32-key block. On return s holds the weights
// e = exp(s - m) and sd holds e * dS_raw (the raw, unscaled score tangent).
// Returns true when the accumulators must be multiplied by `alpha`.
__device__ inline bool softmax_block(f32x16& s, f32x16& sd, RowState& st, float cx, float thr,
                                     float& alpha) {
  float bm = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) bm = fmaxf(bm, s[r]);
  bm = fmaxf(bm, __shfl_xor(bm, 32));
  const bool need = bm > st.m + thr;
  bool rescale = false;
  alpha = 1.0f;
  if (__any(need)) {
    const float mn = fmaxf(st.m, bm);
    alpha = mn == -INFINITY ? 1.0f : exp2f((st.m - mn) * cx);
    st.l *= alpha;
    st.mu *= alpha;
    st.m = mn;
    st.moff = mn == -INFINITY ? 0.0f : mn * cx;
    rescale = true;
  }
  float l = 0.0f, mu = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float e = __builtin_amdgcn_exp2f(fmaf(s[r], cx, -st.moff));
    s[r] = e;
    const float u = e * sd[r];
    sd[r] = u;
    l += e;
    mu += u;
  }
  st.l += l;
  st.mu += mu;
  return rescale;
}

// ------------------------------------------------------------- 16-bit kernel

template <typename T, int D, int MASK, bool CAUSAL>
__global__ __launch_bounds__(kThreads, D == 64 ? 2 : 1) void fwd16_kernel(FwdArgs a) {
  using L = Tile16<D>;
  using vec8 = typename T::vec8;
  __shared__ __attribute__((aligned(16))) char smem[2 * L::BUF_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c32 = lane & 31;
  const int hlf = lane >> 5;

  // Heaviest query blocks first (causal work grows with the block index).
  const int qb = a.n_qblk - 1 - int(blockIdx.x) / a.BH;
  const int bh = int(blockIdx.x) % a.BH;
  const int b = bh / a.H, h = bh % a.H;
  const int q0 = qb * kBM;
  const int qw0 = q0 + 32 * wave;
  const int qi = qw0 + c32;
  const bool wave_live = qw0 < a.Nq;

  const uint16_t* qp = static_cast<const uint16_t*>(a.q) + int64_t(bh) * a.Nq * D;
  const uint16_t* tqp = a.tq ? static_cast<const uint16_t*>(a.tq) + int64_t(bh) * a.Nq * D : nullptr;
  const uint16_t* kp = static_cast<const uint16_t*>(a.k) + int64_t(bh) * a.Nk * D;
  const uint16_t* vp = static_cast<const uint16_t*>(a.v) + int64_t(bh) * a.Nk * D;
  const uint16_t* tkp = a.tk ? static_cast<const uint16_t*>(a.tk) + int64_t(bh) * a.Nk * D : nullptr;
  const uint16_t* tvp = a.tv ? static_cast<const uint16_t*>(a.tv) + int64_t(bh) * a.Nk * D : nullptr;

  // Q and dQ as B operands: lane holds row qi, head-dim entries hlf*D/2 + 8c .. +7.
  vec8 qB[L::NC], tqB[L::NC];
  {
    const bool ok = qi < a.Nq;
#pragma unroll
    for (int c = 0; c < L::NC; ++c) {
      const int64_t off = int64_t(qi) * D + hlf * (D / 2) + 8 * c;
      uint4 x = ok ? *reinterpret_cast<const uint4*>(qp + off) : uint4{0, 0, 0, 0};
      uint4 y = (ok && tqp) ? *reinterpret_cast<const uint4*>(tqp + off) : uint4{0, 0, 0, 0};
      qB[c] = __builtin_bit_cast(vec8, x);
      tqB[c] = __builtin_bit_cast(vec8, y);
    }
  }

  f32x16 accO[L::NT], accT[L::NT];
#pragma unroll
  for (int t = 0; t < L::NT; ++t) {
    accO[t] = f32x16{};
    accT[t] = f32x16{};
  }
  RowState st{-INFINITY, 0.0f, 0.0f, 0.0f};

  const int kv_end = CAUSAL ? min(a.Nk, q0 + kBM) : a.Nk;
  const int n_tiles = (kv_end + L::BN - 1) / L::BN;

  // Staging registers for the next tile.
  uint4 kr[2], tkr[2];
  uint2 vr[4], tvr[4];
  const int vdg = tid % (D / 4), vkg = tid / (D / 4);

  auto load_tile = [&](int j) {
    const int kbase = j * L::BN;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int gi = tid + kThreads * i;
      const int row = gi / L::GR, g = gi % L::GR;
      const int key = kbase + row;
      const int64_t off = int64_t(key) * D + 8 * g;
      kr[i] = key < a.Nk ? *reinterpret_cast<const uint4*>(kp + off) : uint4{0, 0, 0, 0};
      tkr[i] = (key < a.Nk && tkp) ? *reinterpret_cast<const uint4*>(tkp + off) : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = kbase + 4 * vkg + r;
      const int64_t off = int64_t(key) * D + 4 * vdg;
      vr[r] = key < a.Nk ? *reinterpret_cast<const uint2*>(vp + off) : uint2{0, 0};
      tvr[r] = (key < a.Nk && tvp) ? *reinterpret_cast<const uint2*>(tvp + off) : uint2{0, 0};
    }
  };
  auto store_tile = [&](int buf) {
    char* base = smem + buf * L::BUF_BYTES;
    char* sk = base;
    char* stk = base + L::TENSOR_BYTES;
    char* sv = base + 2 * L::TENSOR_BYTES;
    char* stv = base + 3 * L::TENSOR_BYTES;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int gi = tid + kThreads * i;
      const int row = gi / L::GR, g = gi % L::GR;
      lds_store<uint4>(sk, k_off<D>(row, g), kr[i]);
      lds_store<uint4>(stk, k_off<D>(row, g), tkr[i]);
    }
    const int pos = key_pos(4 * vkg);
    const int g = pos >> 3, half = (pos >> 2) & 1;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int dd = 4 * vdg + c;
      const int off = vt_off<D>(dd, g) + 8 * half;
      lds_store<uint2>(sv, off, uint2{col_pair(vr[0], vr[1], c), col_pair(vr[2], vr[3], c)});
      lds_store<uint2>(stv, off, uint2{col_pair(tvr[0], tvr[1], c), col_pair(tvr[2], tvr[3], c)});
    }
  };

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    if (j + 1 < n_tiles) load_tile(j + 1);
    const char* base = smem + (j & 1) * L::BUF_BYTES;
    const char* sk = base;
    const char* stk = base + L::TENSOR_BYTES;
    const char* sv = base + 2 * L::TENSOR_BYTES;
    const char* stv = base + 3 * L::TENSOR_BYTES;

    if (wave_live) {
#pragma unroll
      for (int kb = 0; kb < L::KB; ++kb) {
        const int k0 = j * L::BN + kb * 32;
        if (k0 >= kv_end) break;
        if (CAUSAL && k0 > qw0 + 31) break;
        // S^T and dS^T for 32 keys x 32 queries.
        f32x16 s{}, sd{};
#pragma unroll
        for (int c = 0; c < L::NC; ++c) {
          const int off = k_off<D>(kb * 32 + c32, hlf * L::NC + c);
          const vec8 ka = __builtin_bit_cast(vec8, lds_load<uint4>(sk, off));
          const vec8 tka = __builtin_bit_cast(vec8, lds_load<uint4>(stk, off));
          s = T::mfma(ka, qB[c], s);
          sd = T::mfma(tka, qB[c], sd);
          sd = T::mfma(ka, tqB[c], sd);
        }
        const bool elem_mask = (CAUSAL && k0 + 31 > qw0) || (k0 + 32 > a.Nk);
        mask_scores<T, MASK, CAUSAL>(s, a, b, h, qi, k0, hlf, elem_mask);
        float alpha;
        if (softmax_block(s, sd, st, a.cx, a.thr, alpha)) {
#pragma unroll
          for (int t = 0; t < L::NT; ++t) {
            accO[t] *= alpha;
            accT[t] *= alpha;
          }
        }
        // Weights and weights * dS (scaled) as 16-bit B operands, keys 16kc .. 16kc+15.
        vec8 pB[2], uB[2];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          uint4 pw, uw;
          pw.x = T::pack2(s[8 * kc + 0], s[8 * kc + 1]);
          pw.y = T::pack2(s[8 * kc + 2], s[8 * kc + 3]);
          pw.z = T::pack2(s[8 * kc + 4], s[8 * kc + 5]);
          pw.w = T::pack2(s[8 * kc + 6], s[8 * kc + 7]);
          uw.x = T::pack2(sd[8 * kc + 0] * a.scale, sd[8 * kc + 1] * a.scale);
          uw.y = T::pack2(sd[8 * kc + 2] * a.scale, sd[8 * kc + 3] * a.scale);
          uw.z = T::pack2(sd[8 * kc + 4] * a.scale, sd[8 * kc + 5] * a.scale);
          uw.w = T::pack2(sd[8 * kc + 6] * a.scale, sd[8 * kc + 7] * a.scale);
          pB[kc] = __builtin_bit_cast(vec8, pw);
          uB[kc] = __builtin_bit_cast(vec8, uw);
        }
#pragma unroll
        for (int t = 0; t < L::NT; ++t) {
#pragma unroll
          for (int kc = 0; kc < 2; ++kc) {
            const int off = vt_off<D>(32 * t + c32, kb * 4 + kc * 2 + hlf);
            const vec8 va = __builtin_bit_cast(vec8, lds_load<uint4>(sv, off));
            const vec8 tva = __builtin_bit_cast(vec8, lds_load<uint4>(stv, off));
            accO[t] = T::mfma(va, pB[kc], accO[t]);
            accT[t] = T::mfma(va, uB[kc], accT[t]);
            accT[t] = T::mfma(tva, pB[kc], accT[t]);
          }
        }
      }
    }
    if (j + 1 < n_tiles) store_tile((j + 1) & 1);
    __syncthreads();
  }

  // Epilogue: combine the two lane halves of each query column, normalise, store.
  const float l = st.l + __shfl_xor(st.l, 32);
  const float mu = st.mu + __shfl_xor(st.mu, 32);
  if (qi < a.Nq) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const float tl = mu * a.scale * inv;
    uint16_t* op = static_cast<uint16_t*>(a.o) + int64_t(bh) * a.Nq * D + int64_t(qi) * D;
    uint16_t* top = static_cast<uint16_t*>(a.to) + int64_t(bh) * a.Nq * D + int64_t(qi) * D;
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
        *reinterpret_cast<uint2*>(op + dd) = uint2{T::pack2(ov[0], ov[1]), T::pack2(ov[2], ov[3])};
        *reinterpret_cast<uint2*>(top + dd) = uint2{T::pack2(dv[0], dv[1]), T::pack2(dv[2], dv[3])};
      }
    }
    if (hlf == 0) {
      const int64_t ri = int64_t(bh) * a.Nq + qi;
      a.lse[ri] = l > 0.0f ? (st.moff + log2f(l)) * kLn2 : -INFINITY;
      if (a.tlse) a.tlse[ri] = tl;
    }
  }
}

// ------------------------------------------------------------- float32 kernel
//
// Same structure on v_mfma_f32_32x32x2_f32 (float32 products, no rounding of
// the weights). Each product takes 2 entries of the inner dimension: for the
// score products lane half hlf supplies head-dim entry hlf*D/2 + i for
// product i; for the value products, product m contracts over the keys held
// in C register m of each lane half, so P^T and (P dS)^T are used as they are.

template <int D>
struct Tile32 {
  static constexpr int BN = 32;                 // keys per LDS tile
  static constexpr int NT = D / 32;
  static constexpr int GR = D / 4;              // 16-byte granules per K row
  static constexpr int TENSOR_BYTES = BN * D * 4;
  static constexpr int BUF_BYTES = 4 * TENSOR_BYTES;
};

template <int D>
__device__ inline int k32_off(int row, int g) {
  return row * (4 * D) + ((g ^ (row & 7)) << 4);
}
// V^T row = head-dim index, 32 keys (128 bytes, 8 granules).
__device__ inline int vt32_off(int dd, int g) { return dd * 128 + ((g ^ (dd & 7)) << 4); }

template <int D, int MASK, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd32_kernel(FwdArgs a) {
  using L = Tile32<D>;
  extern __shared__ __attribute__((aligned(16))) char smem32[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c32 = lane & 31;
  const int hlf = lane >> 5;

  const int qb = a.n_qblk - 1 - int(blockIdx.x) / a.BH;
  const int bh = int(blockIdx.x) % a.BH;
  const int b = bh / a.H, h = bh % a.H;
  const int q0 = qb * kBM;
  const int qw0 = q0 + 32 * wave;
  const int qi = qw0 + c32;
  const bool wave_live = qw0 < a.Nq;

  const float* qp = static_cast<const float*>(a.q) + int64_t(bh) * a.Nq * D;
  const float* tqp = a.tq ? static_cast<const float*>(a.tq) + int64_t(bh) * a.Nq * D : nullptr;
  const float* kp = static_cast<const float*>(a.k) + int64_t(bh) * a.Nk * D;
  const float* vp = static_cast<const float*>(a.v) + int64_t(bh) * a.Nk * D;
  const float* tkp = a.tk ? static_cast<const float*>(a.tk) + int64_t(bh) * a.Nk * D : nullptr;
  const float* tvp = a.tv ? static_cast<const float*>(a.tv) + int64_t(bh) * a.Nk * D : nullptr;

  float qB[D / 2], tqB[D / 2];
  {
    const bool ok = qi < a.Nq;
#pragma unroll
    for (int i = 0; i < D / 2; i += 4) {
      const int64_t off = int64_t(qi) * D + hlf * (D / 2) + i;
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

  const int kv_end = CAUSAL ? min(a.Nk, q0 + kBM) : a.Nk;
  const int n_tiles = (kv_end + L::BN - 1) / L::BN;
  char* sk = smem32;
  char* stk = smem32 + L::TENSOR_BYTES;
  char* sv = smem32 + 2 * L::TENSOR_BYTES;
  char* stv = smem32 + 3 * L::TENSOR_BYTES;

  for (int j = 0; j < n_tiles; ++j) {
    const int kbase = j * L::BN;
    // Global -> LDS. K rows as granules; V transposed element by element.
    for (int gi = tid; gi < L::BN * L::GR; gi += kThreads) {
      const int row = gi / L::GR, g = gi % L::GR;
      const int key = kbase + row;
      const int64_t off = int64_t(key) * D + 4 * g;
      const bool ok = key < a.Nk;
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
      mask_scores<F16, MASK == JVPATTN_MASK_ADDITIVE ? -1 : MASK, CAUSAL>(s, a, b, h, qi, k0, hlf,
                                                                          elem_mask);
      if constexpr (MASK == JVPATTN_MASK_ADDITIVE) {
        // float32 additive mask: element (qi, key) for the 16 keys of this lane
        const bool row_ok = qi < a.Nq;
        const float* mp = static_cast<const float*>(a.mask) + b * a.msb + h * a.msh + int64_t(qi) * a.msq;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + (r >> 2) * 8 + 4 * hlf + (r & 3);
          const float mv = (row_ok && key < a.Nk) ? mp[key] : 0.0f;
          s[r] = fmaf(s[r], a.scale, mv);   // hidden keys are already -inf
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

  const float l = st.l + __shfl_xor(st.l, 32);
  const float mu = st.mu + __shfl_xor(st.mu, 32);
  if (qi < a.Nq) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const float tl = mu * a.scale * inv;
    float* op = static_cast<float*>(a.o) + int64_t(bh) * a.Nq * D + int64_t(qi) * D;
    float* top = static_cast<float*>(a.to) + int64_t(bh) * a.Nq * D + int64_t(qi) * D;
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
        *reinterpret_cast<f32x4*>(op + dd) = ov;
        *reinterpret_cast<f32x4*>(top + dd) = dv;
      }
    }
    if (hlf == 0) {
      const int64_t ri = int64_t(bh) * a.Nq + qi;
      a.lse[ri] = l > 0.0f ? (st.moff + log2f(l)) * kLn2 : -INFINITY;
      if (a.tlse) a.tlse[ri] = tl;
    }
  }
}

// ---------------------------------------------------------------- dispatch

thread_local int g_last_hip_error = 0;

template <int MASK, bool CAUSAL>
hipError_t launch_typed(int dtype, int d, const FwdArgs& args, dim3 grid, hipStream_t stream) {
  const dim3 block(kThreads);
  if (dtype == JVPATTN_BF16) {
    if (d == 64) hipLaunchKernelGGL((fwd16_kernel<BF16, 64, MASK, CAUSAL>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((fwd16_kernel<BF16, 128, MASK, CAUSAL>), grid, block, 0, stream, args);
  } else if (dtype == JVPATTN_F16) {
    if (d == 64) hipLaunchKernelGGL((fwd16_kernel<F16, 64, MASK, CAUSAL>), grid, block, 0, stream, args);
    else hipLaunchKernelGGL((fwd16_kernel<F16, 128, MASK, CAUSAL>), grid, block, 0, stream, args);
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
}  // namespace jvpattn

extern "C" int jvpattn_last_hip_error(void) { return jvpattn::g_last_hip_error; }

extern "C" int jvpattn_fwd(const jvpattn_params* p, const void* q, const void* k, const void* v,
                           const void* tq, const void* tk, const void* tv, const void* mask, void* o,
                           void* to, float* lse, float* tlse, void* stream) {
  using namespace jvpattn;
  FwdSizes sz;
  const int rc = check_fwd(p, q, k, v, tq, tk, tv, mask, o, to, lse, tlse, &sz);
  if (rc != JVPATTN_OK) return rc;
  if (sz.rows_q == 0) return JVPATTN_OK;

  FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.tq = tq; a.tk = tk; a.tv = tv; a.mask = mask;
  a.o = o; a.to = to; a.lse = lse; a.tlse = tlse;
  a.H = p->H; a.Nq = p->Nq; a.Nk = p->Nk; a.BH = p->B * p->H;
  a.n_qblk = (p->Nq + kBM - 1) / kBM;
  a.msb = p->mask_stride_b; a.msh = p->mask_stride_h; a.msq = p->mask_stride_q;
  a.scale = p->scale;
  const bool additive = p->mask_kind == JVPATTN_MASK_ADDITIVE;
  // Scores stay raw (q.k) without an additive mask, so scale folds into cx.
  a.cx = additive ? kLog2e : p->scale * kLog2e;
  const float tau = p->dtype == JVPATTN_BF16 ? BF16::kTau : p->dtype == JVPATTN_F16 ? F16::kTau : 8.0f;
  a.thr = tau / a.cx;
  {
    const int mes = p->mask_kind == JVPATTN_MASK_BOOL ? 1 : elem_bytes(p->dtype);
    const uintptr_t base = reinterpret_cast<uintptr_t>(mask);
    const int64_t need = 4;  // keys per vector read
    a.mask_vec = mask && (p->mask_stride_b % need == 0) && (p->mask_stride_h % need == 0) &&
                 (p->mask_stride_q % need == 0) && (base % (need * mes) == 0);
  }
  const int64_t blocks = int64_t(a.n_qblk) * a.BH;
  if (blocks > INT32_MAX) return JVPATTN_ERR_SHAPE;
  const dim3 grid(static_cast<unsigned>(blocks));
  hipStream_t s = static_cast<hipStream_t>(stream);

  hipError_t e;
  const bool c = p->causal != 0;
  switch (p->mask_kind) {
    case JVPATTN_MASK_NONE:
      e = c ? launch_typed<JVPATTN_MASK_NONE, true>(p->dtype, p->d, a, grid, s)
            : launch_typed<JVPATTN_MASK_NONE, false>(p->dtype, p->d, a, grid, s);
      break;
    case JVPATTN_MASK_BOOL:
      e = c ? launch_typed<JVPATTN_MASK_BOOL, true>(p->dtype, p->d, a, grid, s)
            : launch_typed<JVPATTN_MASK_BOOL, false>(p->dtype, p->d, a, grid, s);
      break;
    default:
      e = c ? launch_typed<JVPATTN_MASK_ADDITIVE, true>(p->dtype, p->d, a, grid, s)
            : launch_typed<JVPATTN_MASK_ADDITIVE, false>(p->dtype, p->d, a, grid, s);
      break;
  }
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return JVPATTN_ERR_HIP;
  }
  return JVPATTN_OK;
}
