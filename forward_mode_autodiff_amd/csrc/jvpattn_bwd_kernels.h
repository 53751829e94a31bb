// Reverse pass of the fused attention forward with tangents, for gfx950:
// device code (kernels and their launcher).
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
//   dkv:  one workgroup per 128 keys, looping over 32-query tiles;
//   dq:   one workgroup per 128 queries, looping over 32-key tiles.
// Both tile kernels use the forward's MFMA layout (32x32x16 products, C
// registers rounded to 16 bits reused as B operands, transpose reads of the
// LDS tiles for the accumulating products).
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "jvpattn.h"
#include "jvpattn_bwd_launch.h"
#include "jvpattn_device.h"

namespace jvpattn {
namespace {

static_assert(kBThreads == kTileThreads, "LDS tiles are laid out for 4 waves");



// ------------------------------------------------------------------ rows
// d/8 lanes per query row (one 16-byte granule of each tensor per lane), so a
// wave reads 1 KB of each tensor contiguously; the row's partial sums meet in
// log2(d/8) butterfly exchanges.
template <typename T, int D>
__device__ __forceinline__ void bwd_rows_body(const BwdArgs& a, int64_t rows) {
  constexpr int LPR = D / 8;   // lanes per row
  const int64_t t = int64_t(blockIdx.x) * kBThreads + threadIdx.x;
  const int64_t row = t / LPR;
  const int gi = threadIdx.x % LPR;
  const bool live = row < rows;
  const int64_t at = live ? row * LPR + gi : 0;
  const uint4 wo = live ? static_cast<const uint4*>(a.o)[at] : uint4{0, 0, 0, 0};
  const uint4 wto = live ? static_cast<const uint4*>(a.to)[at] : uint4{0, 0, 0, 0};
  // a NULL cotangent is zero
  const uint4 wg = (live && a.go) ? static_cast<const uint4*>(a.go)[at] : uint4{0, 0, 0, 0};
  const uint4 wgd = (live && a.gto) ? static_cast<const uint4*>(a.gto)[at] : uint4{0, 0, 0, 0};
  const uint32_t xo[4] = {wo.x, wo.y, wo.z, wo.w}, xto[4] = {wto.x, wto.y, wto.z, wto.w};
  const uint32_t xg[4] = {wg.x, wg.y, wg.z, wg.w}, xgd[4] = {wgd.x, wgd.y, wgd.z, wgd.w};
  float r = 0.0f, go_o = 0.0f, gd_to = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int hw = 0; hw < 2; ++hw) {
      const uint16_t so = hw ? hi16(xo[i]) : lo16(xo[i]);
      const uint16_t sto = hw ? hi16(xto[i]) : lo16(xto[i]);
      const uint16_t sg = hw ? hi16(xg[i]) : lo16(xg[i]);
      const uint16_t sgd = hw ? hi16(xgd[i]) : lo16(xgd[i]);
      const float fo = T::widen(so), fgd = T::widen(sgd);
      r = fmaf(fgd, fo, r);
      go_o = fmaf(T::widen(sg), fo, go_o);
      gd_to = fmaf(fgd, T::widen(sto), gd_to);
    }
  }
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) {
    r += __shfl_xor(r, m, LPR);
    go_o += __shfl_xor(go_o, m, LPR);
    gd_to += __shfl_xor(gd_to, m, LPR);
  }
  if (!live || gi != 0) return;
  const float lse = a.lse[row], tl = a.tlse[row];
  a.ws[WS_NEGL * a.ws_stride + row] = lse == -INFINITY ? -INFINITY : -lse * kLog2e;
  a.ws[WS_TLSE * a.ws_stride + row] = tl;
  a.ws[WS_R * a.ws_stride + row] = r;
  a.ws[WS_DEL * a.ws_stride + row] = go_o + gd_to - tl * r;
}

template <typename T, int D>
__global__ __launch_bounds__(kBThreads) void bwd_rows_kernel(BwdArgs a, int64_t rows) {
#if defined(__HIP_DEVICE_COMPILE__)
  bwd_rows_body<T, D>(a, rows);
#endif
}

// Element-wise step shared by both tile kernels. For one score element:
// s (masked score, score units), sd (score tangent, times us gives dS),
// x = (G V^T + Gd dV^T), dm = D, and the row's statistics.
struct Cot {
  float p, pd, sbar, sdbar;
};
__device__ inline Cot cotangents(float s, float sd, float x, float dm, float cx, float us, float negl, float tl,
                                 float r, float del) {
  Cot c;
  c.p = __builtin_amdgcn_exp2f(fmaf(s, cx, negl));
  const float sdv = sd * us;        // dS
  const float sdu = sdv - tl;       // dS - tlse
  c.pd = c.p * sdu;
  const float dp = x + dm * sdu - r * sdv;
  c.sbar = c.p * (dp - del);
  c.sdbar = c.p * (dm - r);
  return c;
}

// ------------------------------------------------------------------ dq
//
// Four waves, 32 queries each (128 per workgroup), a loop over 32-key tiles
// of K, dK, V, dV in the forward's LDS format (ring of 4, fetched two tiles
// ahead). Per tile and wave, with the forward's transposed layout (lane =
// query column, 16 keys per lane):
//   S^T = K Q^T, Sd^T = dK Q^T + K dQ^T, X^T = V G^T + dV Gd^T, D^T = V Gd^T
// (24 products), the cotangents per element, then
//   dq^T += K^T Sbar^T + dK^T Sdbar^T,  dtq^T += K^T Sdbar^T  (12 products).
// PIPE (d = 64 only): the score-side products of the next block overlap the
// current block's element-wise step, at one wave per SIMD; without it blocks
// go one at a time, and at d = 64 that fits two waves per SIMD (two
// workgroups per CU: bwd_dq2_kernel). At d = 128 two blocks' products would
// not fit the registers.
template <typename T, int D, int MASK, bool CAUSAL, bool POW2, bool PIPE = (D == 64)>
__device__ __forceinline__ void bwd_dq_body(const BwdArgs& a) {
  using L = Tile16<D>;
  static_assert(!PIPE || D == 64, "the pipelined query side is built for d = 64");
  using vec8 = typename T::vec8;
  __shared__ __attribute__((aligned(16))) char stage0[L::STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) char stage1[L::STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) char stage2[L::STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) char stage3[L::STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31;
  const int hlf = lane >> 5;

  const int qb = a.n_blk - 1 - int(blockIdx.x) / a.BH;   // heaviest first when causal
  const int bh = int(blockIdx.x) % a.BH;
  const int b = bh / a.H, h = bh % a.H;
  const int q0 = qb * kBBlk;
  const int qw0 = q0 + 32 * wave;
  const int qi = qw0 + c32;
  const bool wave_live = qw0 < a.Nq;

  const int64_t qhead = int64_t(bh) * a.Nq * L::ROW;
  const int64_t khead = int64_t(bh / a.grp) * a.Nk * L::ROW;   // the key/value head it reads
  const int64_t qbytes = int64_t(a.Nq) * L::ROW, kbytes = int64_t(a.Nk) * L::ROW;
  auto at = [](const void* p, int64_t off) { return static_cast<const char*>(p) + off; };

  // B operands of this wave's 32 queries: Q, dQ (scale folded in when exact), G, Gd.
  vec8 qB[L::NC], tqB[L::NC], gB[L::NC], tgB[L::NC];
  {
    const Rsrc rq = make_rsrc(at(a.q, qhead), qbytes);
    const Rsrc rtq = make_rsrc(a.tq ? at(a.tq, qhead) : at(a.q, qhead), a.tq ? qbytes : 0);
    const Rsrc rg = make_rsrc(a.go ? at(a.go, qhead) : at(a.q, qhead), a.go ? qbytes : 0);
    const Rsrc rtg = make_rsrc(a.gto ? at(a.gto, qhead) : at(a.q, qhead), a.gto ? qbytes : 0);
#pragma unroll
    for (int c = 0; c < L::NC; ++c) {
      const int off = qi * L::ROW + (hlf * (D / 2) + 8 * c) * 2;
      qB[c] = __builtin_bit_cast(vec8, ld128(rq, off));
      tqB[c] = __builtin_bit_cast(vec8, ld128(rtq, off));
      gB[c] = __builtin_bit_cast(vec8, ld128(rg, off));
      tgB[c] = __builtin_bit_cast(vec8, ld128(rtg, off));
      if constexpr (POW2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          qB[c][e] = static_cast<__bf16>(static_cast<float>(qB[c][e]) * a.scale);
          tqB[c][e] = static_cast<__bf16>(static_cast<float>(tqB[c][e]) * a.scale);
        }
      }
    }
  }
  // Row statistics of this lane's query (rows past Nq read as zero and are never stored).
  float negl = -INFINITY, tl = 0.0f, rr = 0.0f, del = 0.0f;
  if (qi < a.Nq) {
    const int64_t ri = int64_t(bh) * a.Nq + qi;
    negl = a.ws[WS_NEGL * a.ws_stride + ri];
    tl = a.ws[WS_TLSE * a.ws_stride + ri];
    rr = a.ws[WS_R * a.ws_stride + ri];
    del = a.ws[WS_DEL * a.ws_stride + ri];
  }
  const float us = POW2 ? 1.0f : a.scale;

  f32x16 accQ[L::NT], accTQ[L::NT];
#pragma unroll
  for (int t = 0; t < L::NT; ++t) {
    accQ[t] = f32x16{};
    accTQ[t] = f32x16{};
  }
  const Rsrc mr = mask_rsrc(a, b, h, MASK == JVPATTN_MASK_BOOL ? 1 : MASK == JVPATTN_MASK_BITS ? 4 : 2, nullptr,
                            MASK == JVPATTN_MASK_BITS);
  const Rsrc mtr = MASK == kMaskAddT ? mask_rsrc(a, b, h, 2, a.tmask) : mr;
  auto load_mask = [&](MaskVals<MASK>& m, int k0) {
    if constexpr (MASK == kMaskAddT) mask_load_t(m, a, mr, mtr, qi, k0, hlf);
    else mask_load<MASK>(m, a, mr, qi, k0, hlf);
  };

  const int kv_end = CAUSAL ? min(a.Nk, q0 + kBBlk) : a.Nk;
  const int n_tiles = (kv_end + L::BN - 1) / L::BN;
  const int last = !wave_live ? -1 : (CAUSAL ? min(n_tiles - 1, qw0 >> 5) : n_tiles - 1);
  auto needs_keymask = [&](int k) { return (CAUSAL && k * 32 + 31 > qw0) || (k * 32 + 32 > a.Nk); };

  int dl_off[L::LOADS];
#pragma unroll
  for (int i = 0; i < L::LOADS; ++i) {
    const int p = i * kBThreads + tid;
    const int row = p / L::GR, pg = p % L::GR;
    dl_off[i] = row * L::ROW + ((pg ^ swz(row)) << 4);
  }
  const Rsrc rk = make_rsrc(at(a.k, khead), kbytes), rv = make_rsrc(at(a.v, khead), kbytes);
  const Rsrc rtk = make_rsrc(a.tk ? at(a.tk, khead) : at(a.k, khead), a.tk ? kbytes : 0);
  const Rsrc rtv = make_rsrc(a.tv ? at(a.tv, khead) : at(a.v, khead), a.tv ? kbytes : 0);
  auto issue_tile = [&](int j, char* stage) {
#pragma unroll
    for (int i = 0; i < L::LOADS; ++i) {
      const int off = j * L::TENSOR_BYTES + dl_off[i];
      const int slot = (i * kBThreads + wave * 64) * 16;
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
  // A operands (rows = keys) of tensor `tsr` of the tile at sb.
  auto read_rows = [&](const char* sb, int tsr, vec8 (&x)[L::NC]) {
#pragma unroll
    for (int c = 0; c < L::NC; ++c) x[c] = __builtin_bit_cast(vec8, lds_load<uint4>(sb + tsr * L::TENSOR_BYTES, kofs[c]));
  };
  // Transposed A operands (rows = head dimension, keys along k) of tensor `tsr`.
  auto read_tr = [&](const char* sb, int tsr, vec8 (&x)[L::NT][2]) {
    const char* base = sb + tsr * L::TENSOR_BYTES;
#pragma unroll
    for (int t = 0; t < L::NT; ++t)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const int o0 = 16 * kc * L::ROW + vofs0[t], o1 = 16 * kc * L::ROW + vofs1[t];
        x[t][kc] = __builtin_bit_cast(
            vec8, __builtin_shufflevector(lds_read_tr(base + o0), lds_read_tr(base + o1), 0, 1, 2, 3, 4, 5, 6, 7));
      }
  };

  // Score-side products of the tile at sb: S^T, dS^T (scores), X^T, D^T (value side).
  struct SPh {
    f32x16 s, sd, x, dm;
  };
  auto sphase = [&](const char* sb, SPh& o) {
    vec8 ka[L::NC], tka[L::NC];
    read_rows(sb, 0, ka);
    read_rows(sb, 1, tka);
    o.s = f32x16{};
    o.sd = f32x16{};
    o.x = f32x16{};
    o.dm = f32x16{};
#pragma unroll
    for (int c = 0; c < L::NC; ++c) {
      o.s = T::mfma(ka[c], qB[c], o.s);
      o.sd = T::mfma(tka[c], qB[c], o.sd);
      o.sd = T::mfma(ka[c], tqB[c], o.sd);
    }
    vec8 va[L::NC], tva[L::NC];
    read_rows(sb, 2, va);
    read_rows(sb, 3, tva);
#pragma unroll
    for (int c = 0; c < L::NC; ++c) {
      o.x = T::mfma(va[c], gB[c], o.x);
      o.x = T::mfma(tva[c], tgB[c], o.x);
      o.dm = T::mfma(va[c], tgB[c], o.dm);
    }
  };
  // Element-wise step of block k: score cotangents as 16-bit B operands.
  auto vphase = [&](int k, SPh& p, const MaskVals<MASK>& mk, bool keymask, vec8 (&sB)[2], vec8 (&sdB)[2]) {
    mask_apply<T, MASK, POW2>(p.s, mk, a.scale);
    mask_tangent<T, MASK>(p.sd, mk, POW2 ? 1.0f : a.inv_scale);
    if (keymask) hide_keys<CAUSAL>(p.s, a.Nk, qi, k * 32, hlf);
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      uint32_t w0[4], w1[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r0 = 8 * kc + 2 * i;
        const Cot c0 = cotangents(p.s[r0], p.sd[r0], p.x[r0], p.dm[r0], a.cx, us, negl, tl, rr, del);
        const Cot c1 = cotangents(p.s[r0 + 1], p.sd[r0 + 1], p.x[r0 + 1], p.dm[r0 + 1], a.cx, us, negl, tl, rr, del);
        w0[i] = T::pack2(c0.sbar, c1.sbar);
        w1[i] = T::pack2(c0.sdbar, c1.sdbar);
      }
      sB[kc] = __builtin_bit_cast(vec8, uint4{w0[0], w0[1], w0[2], w0[3]});
      sdB[kc] = __builtin_bit_cast(vec8, uint4{w1[0], w1[1], w1[2], w1[3]});
    }
  };
  // Accumulating products with K^T, dK^T of the tile at sb.
  auto aphase = [&](const char* sb, const vec8 (&sB)[2], const vec8 (&sdB)[2]) {
    vec8 kt[L::NT][2], tkt[L::NT][2];
    read_tr(sb, 0, kt);
    read_tr(sb, 1, tkt);
#pragma unroll
    for (int t = 0; t < L::NT; ++t)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        accQ[t] = T::mfma(kt[t][kc], sB[kc], accQ[t]);
        accQ[t] = T::mfma(tkt[t][kc], sdB[kc], accQ[t]);
        accTQ[t] = T::mfma(kt[t][kc], sdB[kc], accTQ[t]);
      }
  };

  // Blocks 1.. that need per-key masking start at jm: the causal diagonal, a
  // ragged last tile, or the end of this wave's range.
  int jm = last + 1;
  if (CAUSAL) jm = min(jm, qw0 >> 5);
  jm = min(jm, a.Nk >> 5);
  jm = max(jm, 1);

  // Pipelined block k (block k+1 needs no key mask): the score-side products
  // of block k+1 run on the matrix cores while the vector units turn block k
  // into cotangents; block k's accumulating products follow. Tiles are
  // fetched three blocks ahead into a ring of 4.
  auto fast = [&](int k, const char* cur, const char* nxt, char* dma, SPh& pc, SPh& pn, MaskVals<MASK>& mc,
                  MaskVals<MASK>& mn) {
    if (k + 2 < n_tiles) wait_vmcnt<L::TILE_VMEM>();   // tile k+1 (tile k+2 may stay in flight)
    else wait_vmcnt<0>();
    ring_barrier();
    load_mask(mn, (k + 1) * 32);
    if (k + 3 < n_tiles) issue_tile(k + 3, dma);
    sphase(nxt, pn);
    vec8 sB[2], sdB[2];
    vphase(k, pc, mc, false, sB, sdB);
    aphase(cur, sB, sdB);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * L::NC, 0);   // K / dK rows of block k+1
#pragma unroll
    for (int i = 0; i < 3 * L::NC; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // score products
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);          // cotangents of block k
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * L::NC, 0);   // V / dV rows of block k+1
#pragma unroll
    for (int i = 0; i < 3 * L::NC; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // value-side products
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);          // cotangents of block k
    }
  };

  // Prologue: tiles 0..2 in flight; wait for tile 0; block 0's score-side
  // products if it needs no key mask.
  if (n_tiles > 0) issue_tile(0, stage0);
  if (n_tiles > 1) issue_tile(1, stage1);
  if (n_tiles > 2) issue_tile(2, stage2);
  if (n_tiles > 2) wait_vmcnt<2 * L::TILE_VMEM>();
  else if (n_tiles > 1) wait_vmcnt<L::TILE_VMEM>();
  else wait_vmcnt<0>();
  ring_barrier();
  SPh pa, pb;
  MaskVals<MASK> mka, mkb;
  bool ready = false;   // pa holds the current block's score-side products
  if (PIPE && 0 <= last && !needs_keymask(0)) {
    sphase(stage0, pa);
    load_mask(mka, 0);
    ready = true;
  }
  const int kfast = ready ? jm - 1 : 0;   // blocks 0 .. kfast-1 are pipelined
  int k = 0;
  if constexpr (PIPE) {
    for (; k + 4 <= kfast; k += 4) {
      fast(k, stage0, stage1, stage3, pa, pb, mka, mkb);
      fast(k + 1, stage1, stage2, stage0, pb, pa, mkb, mka);
      fast(k + 2, stage2, stage3, stage1, pa, pb, mka, mkb);
      fast(k + 3, stage3, stage0, stage2, pb, pa, mkb, mka);
    }
    if (k < kfast) {
      fast(k, stage0, stage1, stage3, pa, pb, mka, mkb);
      if (k + 1 < kfast) fast(k + 1, stage1, stage2, stage0, pb, pa, mkb, mka);
      if (k + 2 < kfast) fast(k + 2, stage2, stage3, stage1, pa, pb, mka, mkb);
    }
    if (kfast & 1) {   // block kfast's products were left in pb
      pa = pb;
      mka = mkb;
    }
  }

  // Remaining blocks (diagonal, ragged tail, barrier-only ones past this
  // wave's rows), one at a time, stage chosen at run time.
  auto stage_of = [&](int i) -> char* {
    i &= 3;
    return i == 0 ? stage0 : i == 1 ? stage1 : i == 2 ? stage2 : stage3;
  };
  for (k = kfast; k < n_tiles; ++k) {
    if (k + 2 < n_tiles) wait_vmcnt<2 * L::TILE_VMEM>();   // tile k (k+1, k+2 may stay in flight)
    else if (k + 1 < n_tiles) wait_vmcnt<L::TILE_VMEM>();
    else wait_vmcnt<0>();
    ring_barrier();
    if (k + 3 < n_tiles) issue_tile(k + 3, stage_of(k + 3));
    if (k > last) continue;
    const char* cur = stage_of(k);
    if (!ready) {
      sphase(cur, pa);
      load_mask(mka, k * 32);
    }
    vec8 sB[2], sdB[2];
    vphase(k, pa, mka, needs_keymask(k), sB, sdB);
    aphase(cur, sB, sdB);
    ready = false;
  }

  if (qi < a.Nq) {
    uint16_t* dq = static_cast<uint16_t*>(a.dq) + int64_t(bh) * a.Nq * D + int64_t(qi) * D;
    uint16_t* dtq = static_cast<uint16_t*>(a.dtq) + int64_t(bh) * a.Nq * D + int64_t(qi) * D;
#pragma unroll
    for (int t = 0; t < L::NT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = 32 * t + 8 * g + 4 * hlf;
        const f32x16& A = accQ[t];
        const f32x16& B = accTQ[t];
        *reinterpret_cast<uint2*>(dq + dd) =
            uint2{T::pack2(A[4 * g] * a.scale, A[4 * g + 1] * a.scale), T::pack2(A[4 * g + 2] * a.scale, A[4 * g + 3] * a.scale)};
        if (a.dtq)
          *reinterpret_cast<uint2*>(dtq + dd) = uint2{T::pack2(B[4 * g] * a.scale, B[4 * g + 1] * a.scale),
                                                      T::pack2(B[4 * g + 2] * a.scale, B[4 * g + 3] * a.scale)};
      }
  }
}

template <typename T, int D, int MASK, bool CAUSAL, bool POW2>
__global__ __launch_bounds__(kBThreads, 1) void bwd_dq_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  bwd_dq_body<T, D, MASK, CAUSAL, POW2>(a);
#endif
}

// d = 64 without the pipeline, two waves per SIMD: for grids of several
// workgroups per CU, where a second workgroup on the CU hides what the
// pipeline hides within one.
template <typename T, int MASK, bool CAUSAL, bool POW2>
__global__ __launch_bounds__(kBThreads, 2) void bwd_dq2_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  bwd_dq_body<T, 64, MASK, CAUSAL, POW2, false>(a);
#endif
}

// ------------------------------------------------------------------ dkv
//
// Four waves, 32 keys each (128 per workgroup), a loop over 32-query tiles of
// Q, dQ, G, Gd (same LDS format) plus the four row statistics of the tile.
// Here lane = key column and 16 queries per lane:
//   S = Q K^T, Sd = dQ K^T + Q dK^T, X = G V^T + Gd dV^T, D = Gd V^T   (24)
//   dk^T += Q^T Sbar + dQ^T Sdbar, dtk^T += Q^T Sdbar,
//   dv^T += G^T P + Gd^T Pd,       dtv^T += Gd^T P                      (24)
// Row r of a lane's C registers is query 8*(r/4) + 4*(lane/32) + r%4.

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// A walking key-side item's B operands (d = 64): four 16-byte LDS reads per
// tensor (K, dK, V, dV rows 32 rows apart), in one block that also waits for
// them. Read through the builtins, the compiler would order them behind
// every outstanding load of the wave (it cannot tell that the direct loads
// which filled the buffer are older than the previous item's stores); the
// caller has already waited for those direct loads.
__device__ inline void read_ops64(const char* p, u32x4 (&o)[16]) {
  const uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(to_lds(p)));
  asm volatile(
      "ds_read_b128 %0, %16\n"
      "ds_read_b128 %1, %16 offset:16\n"
      "ds_read_b128 %2, %16 offset:32\n"
      "ds_read_b128 %3, %16 offset:48\n"
      "ds_read_b128 %4, %16 offset:4096\n"
      "ds_read_b128 %5, %16 offset:4112\n"
      "ds_read_b128 %6, %16 offset:4128\n"
      "ds_read_b128 %7, %16 offset:4144\n"
      "ds_read_b128 %8, %16 offset:8192\n"
      "ds_read_b128 %9, %16 offset:8208\n"
      "ds_read_b128 %10, %16 offset:8224\n"
      "ds_read_b128 %11, %16 offset:8240\n"
      "ds_read_b128 %12, %16 offset:12288\n"
      "ds_read_b128 %13, %16 offset:12304\n"
      "ds_read_b128 %14, %16 offset:12320\n"
      "ds_read_b128 %15, %16 offset:12336\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7]),
        "=&v"(o[8]), "=&v"(o[9]), "=&v"(o[10]), "=&v"(o[11]), "=&v"(o[12]), "=&v"(o[13]), "=&v"(o[14]),
        "=&v"(o[15])
      : "v"(a));   // no memory clobber: it would make the compiler drain the load queue first; as a
                   // volatile asm it stays behind the caller's (volatile) wait for the direct loads
}

// One query tile j (Q, dQ, G, Gd rows; LOADS direct loads per tensor per
// thread) and statistic `wave` of its 32 rows into stage.
template <typename L>
__device__ __forceinline__ void dkv_issue_tile(Rsrc rq, Rsrc rtq, Rsrc rg, Rsrc rtg, Rsrc rstat,
                                               const int (&dl_off)[L::LOADS], int wave, int lane, int j,
                                               char* stage) {
#pragma unroll
  for (int i = 0; i < L::LOADS; ++i) {
    const int off = j * L::TENSOR_BYTES + dl_off[i];
    const int slot = (i * kBThreads + wave * 64) * 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (__attribute__((address_space(3))) void*)to_lds(stage + slot), 16,
                                             off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rtq, (__attribute__((address_space(3))) void*)to_lds(stage + L::TENSOR_BYTES + slot), 16, off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rg, (__attribute__((address_space(3))) void*)to_lds(stage + 2 * L::TENSOR_BYTES + slot), 16, off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rtg, (__attribute__((address_space(3))) void*)to_lds(stage + 3 * L::TENSOR_BYTES + slot), 16, off, 0, 0, 0);
  }
  // 32 floats of statistic `wave` for rows 32j .. 32j+31 (past Nq: zeros)
  if (lane < 8)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rstat, (__attribute__((address_space(3))) void*)to_lds(stage + L::STAGE_BYTES + wave * 128), 16,
        j * 128 + lane * 16, 0, 0, 0);
}

// Mask values (i, key) for this lane's key and the 16 queries of its rows.
template <int MASK> struct MaskCol {};
template <> struct MaskCol<JVPATTN_MASK_BOOL> { uint32_t w[16]; };
template <> struct MaskCol<JVPATTN_MASK_ADDITIVE> { uint32_t w[16]; };

// PART selects the outputs: 0 all four; at d = 128, where the four
// accumulators would not fit the registers beside the operands, one launch
// with PART 1 (dk, dtk: every product) and one with PART 2 (dv, dtv: only
// the weights P and P dS are needed, from S and dS).
enum { kAllParts = 0, kKeyPart = 1, kValuePart = 2 };

// Whether a key-side instance walks several (key block, K/V head) items per
// workgroup: mask-free, d = 64, all four outputs. After its loops an item
// loads the next item's K, dK, V, dV rows into an LDS buffer of their own
// (direct loads, no register destinations) and the first two query tiles of
// its first head; it then stores its gradients with a fixed count of buffer
// stores per wave, so the next item waits only for its own loads.
template <int D, int PART, int MASK>
constexpr bool dkv_walks() {
  return D == 64 && PART == kAllParts && MASK == JVPATTN_MASK_NONE;
}

template <typename T, int D, int PART, int MASK, bool CAUSAL, bool POW2>
__device__ __forceinline__ void bwd_dkv_body(const BwdArgs& a, int item, int next_item, bool loaded) {
  using L = Tile16<D>;
  constexpr bool KP = PART != kValuePart, VP = PART != kKeyPart;
  constexpr bool WALK = dkv_walks<D, PART, MASK>();
  constexpr int kEpStores = 4 * 4 * L::NT;         // dk, dtk, dv, dtv per 4 x 4 tile group
  constexpr int kOpsDma = 32 * L::ROW / 1024;      // direct loads of a wave's 32 rows of one tensor
  using vec8 = typename T::vec8;
  constexpr int STATS = 4 * 32 * 4;                // four statistics of 32 rows
  constexpr int SB = L::STAGE_BYTES + STATS;
  __shared__ __attribute__((aligned(16))) char stage0[SB];
  __shared__ __attribute__((aligned(16))) char stage1[SB];
  __shared__ __attribute__((aligned(16))) char stage2[SB];
  __shared__ __attribute__((aligned(16))) char stage3[SB];
  // a walking item's K, dK, V, dV rows: wave w's 32 keys of tensor i at (4 w + i) * 32 rows
  __shared__ __attribute__((aligned(16))) char ops[WALK ? 4 * kBBlk * L::ROW : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31;
  const int hlf = lane >> 5;

  const int kb = item / a.BHK;   // causal: early key blocks see the most queries
  const int bhk = item % a.BHK;  // key/value head; its query heads are bhk*grp .. +grp-1
  const int b = bhk * a.grp / a.H;
  const int k0 = kb * kBBlk;
  const int kw0 = k0 + 32 * wave;
  const int kj = kw0 + c32;                 // this lane's key
  const bool wave_live = kw0 < a.Nk;

  const int64_t khead = int64_t(bhk) * a.Nk * L::ROW;
  const int64_t qbytes = int64_t(a.Nq) * L::ROW, kbytes = int64_t(a.Nk) * L::ROW;
  auto at = [](const void* p, int64_t off) { return static_cast<const char*>(p) + off; };

  // B operands of this wave's 32 keys: K, dK (scale folded in when exact), V, dV.
  vec8 kB[L::NC], tkB[L::NC], vB[L::NC], tvB[L::NC];
  constexpr int TILE_VMEM = L::TILE_VMEM + 1;   // four tensors + this wave's statistic
  // A walking item's K, dK, V, dV rows (into ops) and its first head's
  // query tiles t_begin, t_begin + 1 (into stages 0, 1), by direct loads.
  auto prefetch = [&](int it) {
    const int kb2 = it / a.BHK, bhk2 = it % a.BHK;
    const int64_t kh2 = int64_t(bhk2) * a.Nk * L::ROW;
    const Rsrc ro2[4] = {make_rsrc(at(a.k, kh2), kbytes),
                         make_rsrc(a.tk ? at(a.tk, kh2) : at(a.k, kh2), a.tk ? kbytes : 0),
                         make_rsrc(at(a.v, kh2), kbytes),
                         make_rsrc(a.tv ? at(a.tv, kh2) : at(a.v, kh2), a.tv ? kbytes : 0)};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < kOpsDma; ++j) {
        const int r = j * (1024 / L::ROW) + lane / (L::ROW / 16), gq = lane % (L::ROW / 16);
        const int off = (kb2 * kBBlk + 32 * wave + r) * L::ROW + 16 * gq;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ro2[i], (__attribute__((address_space(3))) void*)to_lds(ops + (4 * wave + i) * 32 * L::ROW + j * 1024),
            16, off, 0, 0, 0);
      }
    const int bh2 = bhk2 * a.grp;
    const int64_t qh2 = int64_t(bh2) * a.Nq * L::ROW;
    const Rsrc rq2 = make_rsrc(at(a.q, qh2), qbytes);
    const Rsrc rtq2 = make_rsrc(a.tq ? at(a.tq, qh2) : at(a.q, qh2), a.tq ? qbytes : 0);
    const Rsrc rg2 = make_rsrc(a.go ? at(a.go, qh2) : at(a.q, qh2), a.go ? qbytes : 0);
    const Rsrc rtg2 = make_rsrc(a.gto ? at(a.gto, qh2) : at(a.q, qh2), a.gto ? qbytes : 0);
    const Rsrc rstat2 = make_rsrc(a.ws + wave * a.ws_stride + int64_t(bh2) * a.Nq, int64_t(a.Nq) * 4);
    int dl2[L::LOADS];
#pragma unroll
    for (int i = 0; i < L::LOADS; ++i) {
      const int p = i * kBThreads + tid;
      dl2[i] = (p / L::GR) * L::ROW + (((p % L::GR) ^ swz(p / L::GR)) << 4);
    }
    const int n_qt2 = (a.Nq + 31) / 32;
    const int tb2 = CAUSAL ? min(n_qt2, (kb2 * kBBlk) >> 5) : 0;
    if (tb2 < n_qt2) dkv_issue_tile<L>(rq2, rtq2, rg2, rtg2, rstat2, dl2, wave, lane, tb2, stage0);
    if (tb2 + 1 < n_qt2) dkv_issue_tile<L>(rq2, rtq2, rg2, rtg2, rstat2, dl2, wave, lane, tb2 + 1, stage1);
  };
  if constexpr (WALK) {
    // The first item fetches its own operands and tiles; later ones came with
    // the previous item, ahead of its kEpStores stores, which may stay in
    // flight. Tile t_begin + 1 may stay in flight too (with one query tile
    // only, every load must have landed).
    if (!loaded) prefetch(item);
    const int n_qt0 = (a.Nq + 31) / 32;
    const bool two = n_qt0 - (CAUSAL ? min(n_qt0, k0 >> 5) : 0) > 1;
    if (loaded) {
      if (two) wait_vmcnt<TILE_VMEM + kEpStores>();
      else wait_vmcnt<kEpStores>();
    } else {
      if (two) wait_vmcnt<TILE_VMEM>();
      else wait_vmcnt<0>();
    }
    static_assert(32 * L::ROW == 4096, "read_ops64 takes tensors 4 KB apart");
    u32x4 o[16];
    read_ops64(ops + wave * 4 * 32 * L::ROW + c32 * L::ROW + hlf * (L::ROW / 2), o);
#pragma unroll
    for (int c = 0; c < L::NC; ++c) {
      kB[c] = __builtin_bit_cast(vec8, o[c]);
      tkB[c] = __builtin_bit_cast(vec8, o[4 + c]);
      vB[c] = __builtin_bit_cast(vec8, o[8 + c]);
      tvB[c] = __builtin_bit_cast(vec8, o[12 + c]);
      if constexpr (POW2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kB[c][e] = static_cast<__bf16>(static_cast<float>(kB[c][e]) * a.scale);
          tkB[c][e] = static_cast<__bf16>(static_cast<float>(tkB[c][e]) * a.scale);
        }
      }
    }
  } else {
    const Rsrc rk = make_rsrc(at(a.k, khead), kbytes), rv = make_rsrc(at(a.v, khead), kbytes);
    const Rsrc rtk = make_rsrc(a.tk ? at(a.tk, khead) : at(a.k, khead), a.tk ? kbytes : 0);
    const Rsrc rtv = make_rsrc(a.tv ? at(a.tv, khead) : at(a.v, khead), a.tv ? kbytes : 0);
#pragma unroll
    for (int c = 0; c < L::NC; ++c) {
      const int off = kj * L::ROW + (hlf * (D / 2) + 8 * c) * 2;
      kB[c] = __builtin_bit_cast(vec8, ld128(rk, off));
      tkB[c] = __builtin_bit_cast(vec8, ld128(rtk, off));
      vB[c] = __builtin_bit_cast(vec8, ld128(rv, off));
      tvB[c] = __builtin_bit_cast(vec8, ld128(rtv, off));
      if constexpr (POW2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kB[c][e] = static_cast<__bf16>(static_cast<float>(kB[c][e]) * a.scale);
          tkB[c][e] = static_cast<__bf16>(static_cast<float>(tkB[c][e]) * a.scale);
        }
      }
    }
  }
  const float us = POW2 ? 1.0f : a.scale;

  f32x16 accK[L::NT], accTK[L::NT], accV[L::NT], accTV[L::NT];
#pragma unroll
  for (int t = 0; t < L::NT; ++t) {
    accK[t] = f32x16{};
    accTK[t] = f32x16{};
    accV[t] = f32x16{};
    accTV[t] = f32x16{};
  }
  // Grouped key/value heads: the cotangents of this head's keys sum over the
  // grp query heads that read them, one after the other (the tile pipeline
  // drains and restarts at each change of query head).
  for (int g = 0; g < a.grp; ++g) {
    const int bh = bhk * a.grp + g;
    const int h = bh % a.H;
    const int64_t qhead = int64_t(bh) * a.Nq * L::ROW;
    const Rsrc mr = mask_rsrc(a, b, h, MASK == JVPATTN_MASK_BOOL ? 1 : MASK == JVPATTN_MASK_BITS ? 4 : 2,
                              nullptr, MASK == JVPATTN_MASK_BITS);
    const Rsrc mtr = MASK == kMaskAddT ? mask_rsrc(a, b, h, 2, a.tmask) : mr;

    const int n_qt = (a.Nq + 31) / 32;
    // causal: queries before the block's first key see none of its keys
    const int t_begin = CAUSAL ? min(n_qt, k0 >> 5) : 0;
    const int first = !wave_live ? n_qt : (CAUSAL ? max(t_begin, kw0 >> 5) : 0);   // first tile of this wave
    auto needs_rowmask = [&](int t) { return (CAUSAL && t * 32 < kw0 + 32) || (t * 32 + 32 > a.Nq) || (kw0 + 32 > a.Nk); };

    int dl_off[L::LOADS];
#pragma unroll
    for (int i = 0; i < L::LOADS; ++i) {
      const int p = i * kBThreads + tid;
      const int row = p / L::GR, pg = p % L::GR;
      dl_off[i] = row * L::ROW + ((pg ^ swz(row)) << 4);
    }
    const Rsrc rq = make_rsrc(at(a.q, qhead), qbytes);
    const Rsrc rtq = make_rsrc(a.tq ? at(a.tq, qhead) : at(a.q, qhead), a.tq ? qbytes : 0);
    const Rsrc rg = make_rsrc(a.go ? at(a.go, qhead) : at(a.q, qhead), a.go ? qbytes : 0);
    const Rsrc rtg = make_rsrc(a.gto ? at(a.gto, qhead) : at(a.q, qhead), a.gto ? qbytes : 0);
    // Statistics of this head's rows: wave w loads statistic w of the tile (8 lanes x 16 bytes).
    const int64_t srow = int64_t(bh) * a.Nq;
    const Rsrc rstat = make_rsrc(a.ws + wave * a.ws_stride + srow, int64_t(a.Nq) * 4);
    auto issue_tile = [&](int j, char* stage) { dkv_issue_tile<L>(rq, rtq, rg, rtg, rstat, dl_off, wave, lane, j, stage); };

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
    auto read_rows = [&](const char* sb, int tsr, vec8 (&x)[L::NC]) {
#pragma unroll
      for (int c = 0; c < L::NC; ++c) x[c] = __builtin_bit_cast(vec8, lds_load<uint4>(sb + tsr * L::TENSOR_BYTES, kofs[c]));
    };
    auto read_tr = [&](const char* sb, int tsr, vec8 (&x)[L::NT][2]) {
      const char* base = sb + tsr * L::TENSOR_BYTES;
#pragma unroll
      for (int t = 0; t < L::NT; ++t)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const int o0 = 16 * kc * L::ROW + vofs0[t], o1 = 16 * kc * L::ROW + vofs1[t];
          x[t][kc] = __builtin_bit_cast(
              vec8, __builtin_shufflevector(lds_read_tr(base + o0), lds_read_tr(base + o1), 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };

    auto tile = [&](int t_idx, const char* sb) {
      const int i0 = t_idx * 32;   // first query of the tile
      // Mask elements (query i0 + 8(r/4) + 4 hlf + r%4, key kj) are fetched before the score
      // products so their latency hides behind them (at d = 128, after them: the registers
      // they take are needed by the products' operands).
      uint32_t mw[MASK == JVPATTN_MASK_NONE ? 1 : 16], tw[MASK == kMaskAddT ? 16 : 1];
      auto load_masks = [&]() {
        if constexpr (MASK == JVPATTN_MASK_NONE) return;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qrow = i0 + 8 * (r >> 2) + 4 * hlf + (r & 3);
          if constexpr (MASK == JVPATTN_MASK_BITS) {
            mw[r] = __builtin_amdgcn_raw_buffer_load_b32(mr, (qrow * int(a.msq) + (kj >> 5)) * 4, 0, 0);
          } else if constexpr (MASK == JVPATTN_MASK_BOOL) {
            mw[r] = __builtin_amdgcn_raw_buffer_load_b8(mr, qrow * int(a.msq) + kj, 0, 0);
          } else {
            const int off = (qrow * int(a.msq) + kj) * 2;
            mw[r] = __builtin_amdgcn_raw_buffer_load_b16(mr, off, 0, 0);
            if constexpr (MASK == kMaskAddT) tw[r] = __builtin_amdgcn_raw_buffer_load_b16(mtr, off, 0, 0);
          }
        }
      };
      if constexpr (D == 64) load_masks();
      vec8 qa[L::NC], tqa[L::NC];
      read_rows(sb, 0, qa);
      read_rows(sb, 1, tqa);
      f32x16 s = f32x16{}, sd = f32x16{}, x = f32x16{}, dm = f32x16{};
#pragma unroll
      for (int c = 0; c < L::NC; ++c) {
        s = T::mfma(qa[c], kB[c], s);
        sd = T::mfma(tqa[c], kB[c], sd);
        sd = T::mfma(qa[c], tkB[c], sd);
      }
      if constexpr (D != 64) load_masks();
      if constexpr (KP) {   // X and D enter only the score cotangents
        vec8 ga[L::NC], tga[L::NC];
        read_rows(sb, 2, ga);
        read_rows(sb, 3, tga);
#pragma unroll
        for (int c = 0; c < L::NC; ++c) {
          x = T::mfma(ga[c], vB[c], x);
          x = T::mfma(tga[c], tvB[c], x);
          dm = T::mfma(tga[c], vB[c], dm);
        }
      }
      // masks: element (query i, key kj); hidden entries get score -inf
      if constexpr (MASK == JVPATTN_MASK_BITS) {
#pragma unroll
        for (int r = 0; r < 16; ++r)   // bit kj % 32 of the row's word kj / 32
          if (((mw[r] >> (kj & 31)) & 1u) == 0u) s[r] = -INFINITY;
      } else if constexpr (MASK == JVPATTN_MASK_BOOL) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (mw[r] == 0u) s[r] = -INFINITY;
      } else if constexpr (MASK != JVPATTN_MASK_NONE) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float m = T::widen(uint16_t(mw[r]));
          s[r] = POW2 ? s[r] + m : fmaf(s[r], a.scale, m);
          if constexpr (MASK == kMaskAddT)   // the mask's tangent joins the score tangent (sd * us = dS)
            sd[r] = fmaf(T::widen(uint16_t(tw[r])), POW2 ? 1.0f : a.inv_scale, sd[r]);
        }
      }
      if (needs_rowmask(t_idx)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qrow = i0 + 8 * (r >> 2) + 4 * hlf + (r & 3);
          bool hide = qrow >= a.Nq || kj >= a.Nk;
          if constexpr (CAUSAL) hide = hide || kj > qrow;
          if (hide) s[r] = -INFINITY;
        }
      }
      // statistics of the 16 rows: for group g, rows 8g + 4*hlf + 0..3 (one 16-byte LDS read each)
      const char* st = sb + L::STAGE_BYTES;
      vec8 pB[2], pdB[2], sB[2], sdB[2];
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        uint32_t wp[4], wpd[4], ws[4], wsd[4];
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          const int g = 2 * kc + gg;
          const int roff = (8 * g + 4 * hlf) * 4;
          const f32x4 ng = lds_load<f32x4>(st, WS_NEGL * 128 + roff);
          const f32x4 tl = lds_load<f32x4>(st, WS_TLSE * 128 + roff);
          const f32x4 rr = lds_load<f32x4>(st, WS_R * 128 + roff);
          const f32x4 dl = lds_load<f32x4>(st, WS_DEL * 128 + roff);
          Cot c[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            c[e] = cotangents(s[r], sd[r], x[r], dm[r], a.cx, us, ng[e], tl[e], rr[e], dl[e]);
          }
          wp[2 * gg] = T::pack2(c[0].p, c[1].p);
          wp[2 * gg + 1] = T::pack2(c[2].p, c[3].p);
          wpd[2 * gg] = T::pack2(c[0].pd, c[1].pd);
          wpd[2 * gg + 1] = T::pack2(c[2].pd, c[3].pd);
          ws[2 * gg] = T::pack2(c[0].sbar, c[1].sbar);
          ws[2 * gg + 1] = T::pack2(c[2].sbar, c[3].sbar);
          wsd[2 * gg] = T::pack2(c[0].sdbar, c[1].sdbar);
          wsd[2 * gg + 1] = T::pack2(c[2].sdbar, c[3].sdbar);
        }
        pB[kc] = __builtin_bit_cast(vec8, uint4{wp[0], wp[1], wp[2], wp[3]});
        pdB[kc] = __builtin_bit_cast(vec8, uint4{wpd[0], wpd[1], wpd[2], wpd[3]});
        sB[kc] = __builtin_bit_cast(vec8, uint4{ws[0], ws[1], ws[2], ws[3]});
        sdB[kc] = __builtin_bit_cast(vec8, uint4{wsd[0], wsd[1], wsd[2], wsd[3]});
      }
      if constexpr (KP) {
        vec8 qt[L::NT][2], tqt[L::NT][2];
        read_tr(sb, 0, qt);
        read_tr(sb, 1, tqt);
#pragma unroll
        for (int t = 0; t < L::NT; ++t)
#pragma unroll
          for (int kc = 0; kc < 2; ++kc) {
            accK[t] = T::mfma(qt[t][kc], sB[kc], accK[t]);
            accK[t] = T::mfma(tqt[t][kc], sdB[kc], accK[t]);
            accTK[t] = T::mfma(qt[t][kc], sdB[kc], accTK[t]);
          }
      }
      if constexpr (VP) {
        vec8 gt[L::NT][2], tgt[L::NT][2];
        read_tr(sb, 2, gt);
        read_tr(sb, 3, tgt);
#pragma unroll
        for (int t = 0; t < L::NT; ++t)
#pragma unroll
          for (int kc = 0; kc < 2; ++kc) {
            accV[t] = T::mfma(gt[t][kc], pB[kc], accV[t]);
            accV[t] = T::mfma(tgt[t][kc], pdB[kc], accV[t]);
            accTV[t] = T::mfma(tgt[t][kc], pB[kc], accTV[t]);
          }
      }
    };

    // All waves issue the same count (the statistic load is exec-masked, not skipped).
    // Before step t's wait, tiles t and t+1 may be in flight (t+2 is issued after it).
    auto wait_tile = [&](int j) {
      if (j + 1 < n_qt) wait_vmcnt<TILE_VMEM>();
      else wait_vmcnt<0>();
    };
    const int n_steps = n_qt - t_begin;
    // A walking item's first head has its tiles t_begin, t_begin + 1 in flight already.
    const bool pre = WALK && g == 0;
    if (!pre && n_steps > 0) issue_tile(t_begin, stage0);
    if (!pre && n_steps > 1) issue_tile(t_begin + 1, stage1);
    auto step = [&](int t_idx, const char* cur, char* dma) {
      if (!(pre && t_idx == t_begin)) wait_tile(t_idx);   // else done before the K / V reads
      ring_barrier();
      if (t_idx + 2 < n_qt) issue_tile(t_idx + 2, dma);
      if (t_idx >= first) tile(t_idx, cur);
    };
    for (int i = 0; i < n_steps; i += 4) {
      const int t_idx = t_begin + i;
      step(t_idx, stage0, stage2);
      if (i + 1 < n_steps) step(t_idx + 1, stage1, stage3);
      if (i + 2 < n_steps) step(t_idx + 2, stage2, stage0);
      if (i + 3 < n_steps) step(t_idx + 3, stage3, stage1);
    }
    // every wave is done reading the ring before the next head's loads land in it
    if (g + 1 < a.grp) ring_barrier();
  }

  if (WALK && next_item >= 0) {
    ring_barrier();   // every wave is done with ops and the ring
    prefetch(next_item);
  }

  if constexpr (WALK) {
    // Every wave issues kEpStores stores (keys past Nk land out of range; an
    // absent dtk / dtv has a 0-byte resource).
    const int64_t ob = int64_t(bhk) * a.Nk * D * 2;
    const int64_t ab = int64_t(a.Nk) * D * 2;
    const Rsrc rdk = make_rsrc(static_cast<char*>(a.dk) + ob, ab), rdv = make_rsrc(static_cast<char*>(a.dv) + ob, ab);
    const Rsrc rdtk = make_rsrc(a.dtk ? static_cast<char*>(a.dtk) + ob : static_cast<char*>(a.dk), a.dtk ? ab : 0);
    const Rsrc rdtv = make_rsrc(a.dtv ? static_cast<char*>(a.dtv) + ob : static_cast<char*>(a.dv), a.dtv ? ab : 0);
    const float sc = a.scale;
#pragma unroll
    for (int t = 0; t < L::NT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = 32 * t + 8 * g + 4 * hlf;
        const int e = 4 * g;
        const int off = kj < a.Nk ? (kj * D + dd) * 2 : kOutOfRange;
        st64(rdk, off, uint2{T::pack2(accK[t][e] * sc, accK[t][e + 1] * sc),
                             T::pack2(accK[t][e + 2] * sc, accK[t][e + 3] * sc)});
        st64(rdtk, off, uint2{T::pack2(accTK[t][e] * sc, accTK[t][e + 1] * sc),
                              T::pack2(accTK[t][e + 2] * sc, accTK[t][e + 3] * sc)});
        st64(rdv, off, uint2{T::pack2(accV[t][e], accV[t][e + 1]), T::pack2(accV[t][e + 2], accV[t][e + 3])});
        st64(rdtv, off, uint2{T::pack2(accTV[t][e], accTV[t][e + 1]), T::pack2(accTV[t][e + 2], accTV[t][e + 3])});
      }
  } else if (kj < a.Nk) {
    const int64_t base = int64_t(bhk) * a.Nk * D + int64_t(kj) * D;
    uint16_t* dk = static_cast<uint16_t*>(a.dk) + base;
    uint16_t* dtk = static_cast<uint16_t*>(a.dtk) + base;
    uint16_t* dv = static_cast<uint16_t*>(a.dv) + base;
    uint16_t* dtv = static_cast<uint16_t*>(a.dtv) + base;
    const float sc = a.scale;
#pragma unroll
    for (int t = 0; t < L::NT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = 32 * t + 8 * g + 4 * hlf;
        const int e = 4 * g;
        if constexpr (KP) {
          *reinterpret_cast<uint2*>(dk + dd) = uint2{T::pack2(accK[t][e] * sc, accK[t][e + 1] * sc),
                                                     T::pack2(accK[t][e + 2] * sc, accK[t][e + 3] * sc)};
          if (a.dtk)
            *reinterpret_cast<uint2*>(dtk + dd) = uint2{T::pack2(accTK[t][e] * sc, accTK[t][e + 1] * sc),
                                                        T::pack2(accTK[t][e + 2] * sc, accTK[t][e + 3] * sc)};
        }
        if constexpr (VP) {
          *reinterpret_cast<uint2*>(dv + dd) =
              uint2{T::pack2(accV[t][e], accV[t][e + 1]), T::pack2(accV[t][e + 2], accV[t][e + 3])};
          if (a.dtv)
            *reinterpret_cast<uint2*>(dtv + dd) =
                uint2{T::pack2(accTV[t][e], accTV[t][e + 1]), T::pack2(accTV[t][e + 2], accTV[t][e + 3])};
        }
      }
  }
}

template <typename T, int D, int PART, int MASK, bool CAUSAL, bool POW2>
__global__ __launch_bounds__(kBThreads, 1) void bwd_dkv_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  if constexpr (dkv_walks<D, PART, MASK>()) {
    // Items blockIdx.x + r * gridDim.x, odd rounds reversed within each XCD
    // so heavy and light causal key blocks pair up.
    const int gsz = int(gridDim.x), bx = int(blockIdx.x);
    const int brev = (gsz & 7) == 0 ? (gsz / 8 - 1 - bx / 8) * 8 + (bx & 7) : bx;
    int it = bx;
    for (int r = 0; it < a.n_items; ++r) {
      const int nx = (r + 1) * gsz + ((r & 1) ? bx : brev);
      bwd_dkv_body<T, D, PART, MASK, CAUSAL, POW2>(a, it, nx < a.n_items ? nx : -1, r > 0);
      it = nx;
    }
  } else {
    bwd_dkv_body<T, D, PART, MASK, CAUSAL, POW2>(a, int(blockIdx.x), -1, false);
  }
#endif
}

// ------------------------------------------------------------------ float32
//
// The reverse pass for float32 inputs (d = 64) on v_mfma_f32_32x32x2_f32, in
// the float32 forward's style: each tile is staged through registers into
// one LDS buffer per step (rows, and their transposes for the accumulating
// products), and nothing is rounded below float32. Each product takes two
// entries of its inner dimension per instruction: for the score-side products
// lane half hlf supplies head-dim entry hlf*D/2 + i of product i; for the
// accumulating products, product m contracts over the rows held in C
// register m of each lane half, so the cotangents feed them as they are.

template <int D>
__device__ __forceinline__ void bwd_rows32_body(const BwdArgs& a, int64_t rows) {
  constexpr int LPR = D / 4;   // lanes per row: one float4 of each tensor per lane
  const int64_t t = int64_t(blockIdx.x) * kBThreads + threadIdx.x;
  const int64_t row = t / LPR;
  const int gi = threadIdx.x % LPR;
  const bool live = row < rows;
  const int64_t at = live ? row * LPR + gi : 0;
  const f32x4 z{};
  const f32x4 o = live ? static_cast<const f32x4*>(a.o)[at] : z;
  const f32x4 to = live ? static_cast<const f32x4*>(a.to)[at] : z;
  const f32x4 g = (live && a.go) ? static_cast<const f32x4*>(a.go)[at] : z;   // a NULL cotangent is zero
  const f32x4 gd = (live && a.gto) ? static_cast<const f32x4*>(a.gto)[at] : z;
  float r = 0.0f, go_o = 0.0f, gd_to = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r = fmaf(gd[e], o[e], r);
    go_o = fmaf(g[e], o[e], go_o);
    gd_to = fmaf(gd[e], to[e], gd_to);
  }
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) {
    r += __shfl_xor(r, m, LPR);
    go_o += __shfl_xor(go_o, m, LPR);
    gd_to += __shfl_xor(gd_to, m, LPR);
  }
  if (!live || gi != 0) return;
  const float lse = a.lse[row], tl = a.tlse[row];
  a.ws[WS_NEGL * a.ws_stride + row] = lse == -INFINITY ? -INFINITY : -lse * kLog2e;
  a.ws[WS_TLSE * a.ws_stride + row] = tl;
  a.ws[WS_R * a.ws_stride + row] = r;
  a.ws[WS_DEL * a.ws_stride + row] = go_o + gd_to - tl * r;
}

template <int D>
__global__ __launch_bounds__(kBThreads) void bwd_rows32_kernel(BwdArgs a, int64_t rows) {
#if defined(__HIP_DEVICE_COMPILE__)
  bwd_rows32_body<D>(a, rows);
#endif
}

// One float4 of `p` (row `row`, granule g of D/4), zero past `n` rows or for a NULL tensor.
template <int D>
__device__ inline f32x4 row_granule(const float* p, int row, int n, int g) {
  return (p && row < n) ? *reinterpret_cast<const f32x4*>(p + int64_t(row) * D + 4 * g) : f32x4{};
}

// Rows r0 .. r0+31 of up to four tensors into LDS: as rows (k32 layout) into
// rows[i] and, where tr[i] is set, transposed (vt32 layout) as well.
template <int D, int NTS>
__device__ inline void stage32(const float* const (&src)[NTS], char* const (&rows)[NTS], char* const (&tr)[NTS],
                               int r0, int n) {
  using L = Tile32<D>;
  for (int gi = threadIdx.x; gi < L::BN * L::GR; gi += kBThreads) {
    const int row = gi / L::GR, g = gi % L::GR;
#pragma unroll
    for (int i = 0; i < NTS; ++i) {
      const f32x4 x = row_granule<D>(src[i], r0 + row, n, g);
      lds_store<f32x4>(rows[i], k32_off<D>(row, g), x);
      if (tr[i]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) lds_store<float>(tr[i], vt32_off(4 * g + e, row >> 2) + 4 * (row & 3), x[e]);
      }
    }
  }
}

// dq kernel, float32: four waves of 32 queries, 32-key tiles of K, dK, V, dV
// (rows) and K, dK (transposed); per tile and wave S^T, dS^T, X^T, D^T (the
// forward's transposed layout: lane = query column, 16 keys per lane), the
// cotangents per element, then dq^T += K^T Sbar^T + dK^T Sdbar^T and
// dtq^T += K^T Sdbar^T.
template <int D, int MASK, bool CAUSAL>
__device__ __forceinline__ void bwd_dq32_body(const BwdArgs& a) {
  using L = Tile32<D>;
  constexpr int TB = L::TENSOR_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[6 * TB];
  char* const sk = smem;
  char* const stk = smem + TB;
  char* const sv = smem + 2 * TB;
  char* const stv = smem + 3 * TB;
  char* const skt = smem + 4 * TB;
  char* const stkt = smem + 5 * TB;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c32 = lane & 31;
  const int hlf = lane >> 5;
  const int qb = a.n_blk - 1 - int(blockIdx.x) / a.BH;   // heaviest first when causal
  const int bh = int(blockIdx.x) % a.BH;
  const int b = bh / a.H, h = bh % a.H;
  const int q0 = qb * kBBlk;
  const int qw0 = q0 + 32 * wave;
  const int qi = qw0 + c32;
  const bool wave_live = qw0 < a.Nq;

  const int64_t qhead = int64_t(bh) * a.Nq * D, khead = int64_t(bh / a.grp) * a.Nk * D;
  auto at = [](const void* p, int64_t off) { return p ? static_cast<const float*>(p) + off : nullptr; };
  float qB[D / 2], tqB[D / 2], gB[D / 2], tgB[D / 2];
  {
    const float* src[4] = {at(a.q, qhead), at(a.tq, qhead), at(a.go, qhead), at(a.gto, qhead)};
#pragma unroll
    for (int i = 0; i < D / 2; i += 4) {
      const int g = (hlf * (D / 2) + i) / 4;
      const f32x4 x0 = row_granule<D>(src[0], qi, a.Nq, g), x1 = row_granule<D>(src[1], qi, a.Nq, g);
      const f32x4 x2 = row_granule<D>(src[2], qi, a.Nq, g), x3 = row_granule<D>(src[3], qi, a.Nq, g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qB[i + e] = x0[e];
        tqB[i + e] = x1[e];
        gB[i + e] = x2[e];
        tgB[i + e] = x3[e];
      }
    }
  }
  float negl = -INFINITY, tl = 0.0f, rr = 0.0f, del = 0.0f;
  if (qi < a.Nq) {
    const int64_t ri = int64_t(bh) * a.Nq + qi;
    negl = a.ws[WS_NEGL * a.ws_stride + ri];
    tl = a.ws[WS_TLSE * a.ws_stride + ri];
    rr = a.ws[WS_R * a.ws_stride + ri];
    del = a.ws[WS_DEL * a.ws_stride + ri];
  }

  f32x16 accQ[L::NT], accTQ[L::NT];
#pragma unroll
  for (int t = 0; t < L::NT; ++t) {
    accQ[t] = f32x16{};
    accTQ[t] = f32x16{};
  }
  constexpr bool ADD = MASK == JVPATTN_MASK_ADDITIVE || MASK == kMaskAddT;
  const Rsrc mr = mask_rsrc(a, b, h, mask_es<MASK>(4), nullptr, MASK == JVPATTN_MASK_BITS);
  const Rsrc mtr = MASK == kMaskAddT ? mask_rsrc(a, b, h, 4, a.tmask) : mr;

  const int kv_end = CAUSAL ? min(a.Nk, q0 + kBBlk) : a.Nk;
  const int n_tiles = (kv_end + L::BN - 1) / L::BN;
  const float* const ksrc[4] = {at(a.k, khead), at(a.tk, khead), at(a.v, khead), at(a.tv, khead)};
  char* const krows[4] = {sk, stk, sv, stv};
  char* const ktr[4] = {skt, stkt, nullptr, nullptr};
  for (int j = 0; j < n_tiles; ++j) {
    const int k0 = j * L::BN;
    stage32<D, 4>(ksrc, krows, ktr, k0, a.Nk);
    __syncthreads();
    if (wave_live && !(CAUSAL && k0 > qw0 + 31)) {
      f32x16 s{}, sd{}, x{}, dm{};
#pragma unroll
      for (int i = 0; i < D / 2; i += 4) {
        const int g = (hlf * (D / 2) + i) / 4;
        const f32x4 ka = lds_load<f32x4>(sk, k32_off<D>(c32, g));
        const f32x4 tka = lds_load<f32x4>(stk, k32_off<D>(c32, g));
        const f32x4 va = lds_load<f32x4>(sv, k32_off<D>(c32, g));
        const f32x4 tva = lds_load<f32x4>(stv, k32_off<D>(c32, g));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s = __builtin_amdgcn_mfma_f32_32x32x2f32(ka[e], qB[i + e], s, 0, 0, 0);
          sd = __builtin_amdgcn_mfma_f32_32x32x2f32(tka[e], qB[i + e], sd, 0, 0, 0);
          sd = __builtin_amdgcn_mfma_f32_32x32x2f32(ka[e], tqB[i + e], sd, 0, 0, 0);
          x = __builtin_amdgcn_mfma_f32_32x32x2f32(va[e], gB[i + e], x, 0, 0, 0);
          x = __builtin_amdgcn_mfma_f32_32x32x2f32(tva[e], tgB[i + e], x, 0, 0, 0);
          dm = __builtin_amdgcn_mfma_f32_32x32x2f32(va[e], tgB[i + e], dm, 0, 0, 0);
        }
      }
      // masks: bool / bits / causal / ragged tail hide keys (-inf); additive: s = scale s + m
      if constexpr (!ADD && MASK != JVPATTN_MASK_NONE) {
        MaskVals<MASK> mk;
        mask_load<MASK>(mk, a, mr, qi, k0, hlf);
        mask_apply<F16, MASK, false>(s, mk, a.scale);
      }
      if ((CAUSAL && k0 + 31 > qw0) || (k0 + 32 > a.Nk)) hide_keys<CAUSAL>(s, a.Nk, qi, k0, hlf);
      if constexpr (ADD) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + (r >> 2) * 8 + 4 * hlf + (r & 3);
          const int off = (qi * int(a.msq) + key) * 4;
          s[r] = fmaf(s[r], a.scale, __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(mr, off, 0, 0)));
          if constexpr (MASK == kMaskAddT)   // the mask's tangent joins the score tangent (sd * scale = dS)
            sd[r] = fmaf(__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(mtr, off, 0, 0)), a.inv_scale, sd[r]);
        }
      }
      float sbar[16], sdbar[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const Cot c = cotangents(s[r], sd[r], x[r], dm[r], a.cx, a.scale, negl, tl, rr, del);
        sbar[r] = c.sbar;
        sdbar[r] = c.sdbar;
      }
#pragma unroll
      for (int t = 0; t < L::NT; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int off = vt32_off(32 * t + c32, 2 * g + hlf);
          const f32x4 kt = lds_load<f32x4>(skt, off);
          const f32x4 tkt = lds_load<f32x4>(stkt, off);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int m = 4 * g + e;
            accQ[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(kt[e], sbar[m], accQ[t], 0, 0, 0);
            accQ[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(tkt[e], sdbar[m], accQ[t], 0, 0, 0);
            accTQ[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(kt[e], sdbar[m], accTQ[t], 0, 0, 0);
          }
        }
    }
    __syncthreads();
  }

  if (qi < a.Nq) {
    float* dq = static_cast<float*>(a.dq) + qhead + int64_t(qi) * D;
    float* dtq = a.dtq ? static_cast<float*>(a.dtq) + qhead + int64_t(qi) * D : nullptr;
#pragma unroll
    for (int t = 0; t < L::NT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = 32 * t + 8 * g + 4 * hlf;
        f32x4 u, w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          u[e] = accQ[t][4 * g + e] * a.scale;
          w[e] = accTQ[t][4 * g + e] * a.scale;
        }
        *reinterpret_cast<f32x4*>(dq + dd) = u;
        if (dtq) *reinterpret_cast<f32x4*>(dtq + dd) = w;
      }
  }
}

template <int D, int MASK, bool CAUSAL>
__global__ __launch_bounds__(kBThreads, 1) void bwd_dq32_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  bwd_dq32_body<D, MASK, CAUSAL>(a);
#endif
}

// dkv kernel, float32: four waves of 32 keys, 32-query tiles of Q, dQ, G, Gd
// (rows and transposed) plus the tile's four row statistics; lane = key
// column, 16 queries per lane (row r of a lane's C registers is query
// 8*(r/4) + 4*(lane/32) + r%4): S, dS, X, D, the cotangents, then
// dk^T += Q^T Sbar + dQ^T Sdbar, dtk^T += Q^T Sdbar, dv^T += G^T P + Gd^T Pd,
// dtv^T += Gd^T P. Grouped key/value heads sum over their query heads.
template <int D, int MASK, bool CAUSAL>
__device__ __forceinline__ void bwd_dkv32_body(const BwdArgs& a) {
  using L = Tile32<D>;
  constexpr int TB = L::TENSOR_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[8 * TB];
  __shared__ float stats[4 * 32];
  char* const sq = smem;
  char* const stq = smem + TB;
  char* const sg = smem + 2 * TB;
  char* const stg = smem + 3 * TB;
  char* const sqt = smem + 4 * TB;
  char* const stqt = smem + 5 * TB;
  char* const sgt = smem + 6 * TB;
  char* const stgt = smem + 7 * TB;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c32 = lane & 31;
  const int hlf = lane >> 5;
  const int kb = int(blockIdx.x) / a.BHK;   // causal: early key blocks see the most queries
  const int bhk = int(blockIdx.x) % a.BHK;
  const int b = bhk * a.grp / a.H;
  const int k0 = kb * kBBlk;
  const int kw0 = k0 + 32 * wave;
  const int kj = kw0 + c32;
  const bool wave_live = kw0 < a.Nk;

  const int64_t khead = int64_t(bhk) * a.Nk * D;
  auto at = [](const void* p, int64_t off) { return p ? static_cast<const float*>(p) + off : nullptr; };
  float kB[D / 2], tkB[D / 2], vB[D / 2], tvB[D / 2];
  {
    const float* src[4] = {at(a.k, khead), at(a.tk, khead), at(a.v, khead), at(a.tv, khead)};
#pragma unroll
    for (int i = 0; i < D / 2; i += 4) {
      const int g = (hlf * (D / 2) + i) / 4;
      const f32x4 x0 = row_granule<D>(src[0], kj, a.Nk, g), x1 = row_granule<D>(src[1], kj, a.Nk, g);
      const f32x4 x2 = row_granule<D>(src[2], kj, a.Nk, g), x3 = row_granule<D>(src[3], kj, a.Nk, g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kB[i + e] = x0[e];
        tkB[i + e] = x1[e];
        vB[i + e] = x2[e];
        tvB[i + e] = x3[e];
      }
    }
  }
  f32x16 accK[L::NT], accTK[L::NT], accV[L::NT], accTV[L::NT];
#pragma unroll
  for (int t = 0; t < L::NT; ++t) {
    accK[t] = f32x16{};
    accTK[t] = f32x16{};
    accV[t] = f32x16{};
    accTV[t] = f32x16{};
  }
  constexpr bool ADD = MASK == JVPATTN_MASK_ADDITIVE || MASK == kMaskAddT;

  for (int gq = 0; gq < a.grp; ++gq) {
    const int bh = bhk * a.grp + gq;
    const int h = bh % a.H;
    const int64_t qhead = int64_t(bh) * a.Nq * D;
    const Rsrc mr = mask_rsrc(a, b, h, mask_es<MASK>(4), nullptr, MASK == JVPATTN_MASK_BITS);
    const Rsrc mtr = MASK == kMaskAddT ? mask_rsrc(a, b, h, 4, a.tmask) : mr;
    const int n_qt = (a.Nq + 31) / 32;
    const int t_begin = CAUSAL ? min(n_qt, k0 >> 5) : 0;   // queries before the block see none of its keys
    const int first = !wave_live ? n_qt : (CAUSAL ? max(t_begin, kw0 >> 5) : 0);
    const float* const qsrc[4] = {at(a.q, qhead), at(a.tq, qhead), at(a.go, qhead), at(a.gto, qhead)};
    char* const qrows[4] = {sq, stq, sg, stg};
    char* const qtr[4] = {sqt, stqt, sgt, stgt};
    for (int t = t_begin; t < n_qt; ++t) {
      const int i0 = t * 32;
      stage32<D, 4>(qsrc, qrows, qtr, i0, a.Nq);
      if (tid < 128) {   // statistic tid/32 of row i0 + tid%32 (rows past Nq: 0, never used)
        const int row = i0 + (tid & 31);
        stats[tid] = row < a.Nq ? a.ws[(tid >> 5) * a.ws_stride + int64_t(bh) * a.Nq + row] : 0.0f;
      }
      __syncthreads();
      if (t >= first) {
        f32x16 s{}, sd{}, x{}, dm{};
#pragma unroll
        for (int i = 0; i < D / 2; i += 4) {
          const int g = (hlf * (D / 2) + i) / 4;
          const f32x4 qa = lds_load<f32x4>(sq, k32_off<D>(c32, g));
          const f32x4 tqa = lds_load<f32x4>(stq, k32_off<D>(c32, g));
          const f32x4 ga = lds_load<f32x4>(sg, k32_off<D>(c32, g));
          const f32x4 tga = lds_load<f32x4>(stg, k32_off<D>(c32, g));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[e], kB[i + e], s, 0, 0, 0);
            sd = __builtin_amdgcn_mfma_f32_32x32x2f32(tqa[e], kB[i + e], sd, 0, 0, 0);
            sd = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[e], tkB[i + e], sd, 0, 0, 0);
            x = __builtin_amdgcn_mfma_f32_32x32x2f32(ga[e], vB[i + e], x, 0, 0, 0);
            x = __builtin_amdgcn_mfma_f32_32x32x2f32(tga[e], tvB[i + e], x, 0, 0, 0);
            dm = __builtin_amdgcn_mfma_f32_32x32x2f32(tga[e], vB[i + e], dm, 0, 0, 0);
          }
        }
        // element (query i0 + 8(r/4) + 4 hlf + r%4, key kj)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qrow = i0 + 8 * (r >> 2) + 4 * hlf + (r & 3);
          if constexpr (MASK == JVPATTN_MASK_BITS) {
            const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(mr, (qrow * int(a.msq) + (kj >> 5)) * 4, 0, 0);
            if (((w >> (kj & 31)) & 1u) == 0u) s[r] = -INFINITY;
          } else if constexpr (MASK == JVPATTN_MASK_BOOL) {
            if (__builtin_amdgcn_raw_buffer_load_b8(mr, qrow * int(a.msq) + kj, 0, 0) == 0) s[r] = -INFINITY;
          } else if constexpr (ADD) {
            const int off = (qrow * int(a.msq) + kj) * 4;
            s[r] = fmaf(s[r], a.scale, __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(mr, off, 0, 0)));
            if constexpr (MASK == kMaskAddT)
              sd[r] = fmaf(__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(mtr, off, 0, 0)), a.inv_scale,
                           sd[r]);
          }
          bool hide = qrow >= a.Nq || kj >= a.Nk;
          if constexpr (CAUSAL) hide = hide || kj > qrow;
          if (hide) s[r] = -INFINITY;
        }
        float p[16], pd[16], sbar[16], sdbar[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 8 * (r >> 2) + 4 * hlf + (r & 3);
          const Cot c = cotangents(s[r], sd[r], x[r], dm[r], a.cx, a.scale, stats[WS_NEGL * 32 + row],
                                   stats[WS_TLSE * 32 + row], stats[WS_R * 32 + row], stats[WS_DEL * 32 + row]);
          p[r] = c.p;
          pd[r] = c.pd;
          sbar[r] = c.sbar;
          sdbar[r] = c.sdbar;
        }
#pragma unroll
        for (int tt = 0; tt < L::NT; ++tt)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int off = vt32_off(32 * tt + c32, 2 * g + hlf);
            const f32x4 qt = lds_load<f32x4>(sqt, off);
            const f32x4 tqt = lds_load<f32x4>(stqt, off);
            const f32x4 gt = lds_load<f32x4>(sgt, off);
            const f32x4 tgt = lds_load<f32x4>(stgt, off);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int m = 4 * g + e;
              accK[tt] = __builtin_amdgcn_mfma_f32_32x32x2f32(qt[e], sbar[m], accK[tt], 0, 0, 0);
              accK[tt] = __builtin_amdgcn_mfma_f32_32x32x2f32(tqt[e], sdbar[m], accK[tt], 0, 0, 0);
              accTK[tt] = __builtin_amdgcn_mfma_f32_32x32x2f32(qt[e], sdbar[m], accTK[tt], 0, 0, 0);
              accV[tt] = __builtin_amdgcn_mfma_f32_32x32x2f32(gt[e], p[m], accV[tt], 0, 0, 0);
              accV[tt] = __builtin_amdgcn_mfma_f32_32x32x2f32(tgt[e], pd[m], accV[tt], 0, 0, 0);
              accTV[tt] = __builtin_amdgcn_mfma_f32_32x32x2f32(tgt[e], p[m], accTV[tt], 0, 0, 0);
            }
          }
      }
      __syncthreads();
    }
  }

  if (kj < a.Nk) {
    const int64_t base = khead + int64_t(kj) * D;
    float* dk = static_cast<float*>(a.dk) + base;
    float* dv = static_cast<float*>(a.dv) + base;
    float* dtk = a.dtk ? static_cast<float*>(a.dtk) + base : nullptr;
    float* dtv = a.dtv ? static_cast<float*>(a.dtv) + base : nullptr;
#pragma unroll
    for (int t = 0; t < L::NT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int dd = 32 * t + 8 * g + 4 * hlf;
        f32x4 uk, utk, uv, utv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uk[e] = accK[t][4 * g + e] * a.scale;
          utk[e] = accTK[t][4 * g + e] * a.scale;
          uv[e] = accV[t][4 * g + e];
          utv[e] = accTV[t][4 * g + e];
        }
        *reinterpret_cast<f32x4*>(dk + dd) = uk;
        *reinterpret_cast<f32x4*>(dv + dd) = uv;
        if (dtk) *reinterpret_cast<f32x4*>(dtk + dd) = utk;
        if (dtv) *reinterpret_cast<f32x4*>(dtv + dd) = utv;
      }
  }
}

template <int D, int MASK, bool CAUSAL>
__global__ __launch_bounds__(kBThreads, 1) void bwd_dkv32_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  bwd_dkv32_body<D, MASK, CAUSAL>(a);
#endif
}

// ------------------------------------------------------------------ launch

// WHICH: kLaunchDkv (the rows kernel, then dkv) or kLaunchDq.
template <int WHICH, typename T, int D, int MASK, bool CAUSAL, bool POW2>
hipError_t launch_tiles(BwdArgs a, hipStream_t s) {
  const int64_t nkb = (a.Nk + kBBlk - 1) / kBBlk, nqb = (a.Nq + kBBlk - 1) / kBBlk;
  if (nkb * a.BHK > INT32_MAX || nqb * a.BH > INT32_MAX) return hipErrorInvalidValue;
  if constexpr (WHICH == kLaunchDkv) {
    if (nkb == 0 || a.BHK == 0) return hipSuccess;
    BwdArgs ak = a;
    ak.n_blk = static_cast<int>(nkb);
    ak.n_items = static_cast<int>(nkb * a.BHK);
    if constexpr (D == 64) {
      // the walking instance runs at most a.max_wgs workgroups (a multiple of 8, so each keeps its XCD)
      const int64_t cap = dkv_walks<D, kAllParts, MASK>() ? a.max_wgs : 0;
      const dim3 grid(unsigned(cap > 0 && cap < ak.n_items ? cap : ak.n_items));
      hipLaunchKernelGGL((bwd_dkv_kernel<T, D, kAllParts, MASK, CAUSAL, POW2>), grid, dim3(kBThreads), 0, s, ak);
    } else {
      const dim3 grid(unsigned(ak.n_items));
      hipLaunchKernelGGL((bwd_dkv_kernel<T, D, kKeyPart, MASK, CAUSAL, POW2>), grid, dim3(kBThreads), 0, s, ak);
      hipLaunchKernelGGL((bwd_dkv_kernel<T, D, kValuePart, MASK, CAUSAL, POW2>), grid, dim3(kBThreads), 0, s, ak);
    }
  }
  if constexpr (WHICH == kLaunchDq) {
    if (nqb == 0 || a.BH == 0) return hipSuccess;
    BwdArgs aq = a;
    aq.n_blk = static_cast<int>(nqb);
    const dim3 grid(unsigned(nqb * a.BH));
    bool two = false;
    if constexpr (D == 64) two = a.dq_two != 0;
    if constexpr (D == 64) {
      if (two) hipLaunchKernelGGL((bwd_dq2_kernel<T, MASK, CAUSAL, POW2>), grid, dim3(kBThreads), 0, s, aq);
    }
    if (!two) hipLaunchKernelGGL((bwd_dq_kernel<T, D, MASK, CAUSAL, POW2>), grid, dim3(kBThreads), 0, s, aq);
  }
  return hipGetLastError();
}

template <int WHICH, typename T, int D, int MASK>
hipError_t launch_mask(const BwdArgs& a, bool causal, bool pow2, hipStream_t s) {
  if constexpr (std::is_same_v<T, BF16>) {   // the scale fold is exact only in bfloat16
    if (pow2)
      return causal ? launch_tiles<WHICH, T, D, MASK, true, true>(a, s)
                    : launch_tiles<WHICH, T, D, MASK, false, true>(a, s);
  }
  return causal ? launch_tiles<WHICH, T, D, MASK, true, false>(a, s)
                : launch_tiles<WHICH, T, D, MASK, false, false>(a, s);
}

template <int WHICH, typename T, int D>
hipError_t launch_type(const BwdArgs& a, int mask_kind, bool causal, bool pow2, hipStream_t s) {
  switch (mask_kind) {
    case JVPATTN_MASK_NONE: return launch_mask<WHICH, T, D, JVPATTN_MASK_NONE>(a, causal, pow2, s);
    case JVPATTN_MASK_BOOL: return launch_mask<WHICH, T, D, JVPATTN_MASK_BOOL>(a, causal, pow2, s);
    case JVPATTN_MASK_BITS: return launch_mask<WHICH, T, D, JVPATTN_MASK_BITS>(a, causal, pow2, s);
    case kMaskAddT: return launch_mask<WHICH, T, D, kMaskAddT>(a, causal, pow2, s);
    default: return launch_mask<WHICH, T, D, JVPATTN_MASK_ADDITIVE>(a, causal, pow2, s);
  }
}

}  // namespace

// float32 (d = 64): the same sides with the float32 kernels.
template <int WHICH, int D, int MASK, bool CAUSAL>
hipError_t launch_tiles32(BwdArgs a, hipStream_t s) {
  const int64_t nkb = (a.Nk + kBBlk - 1) / kBBlk, nqb = (a.Nq + kBBlk - 1) / kBBlk;
  if (nkb * a.BHK > INT32_MAX || nqb * a.BH > INT32_MAX) return hipErrorInvalidValue;
  if constexpr (WHICH == kLaunchDkv) {
    if (nkb == 0 || a.BHK == 0) return hipSuccess;
    a.n_blk = static_cast<int>(nkb);
    hipLaunchKernelGGL((bwd_dkv32_kernel<D, MASK, CAUSAL>), dim3(unsigned(nkb * a.BHK)), dim3(kBThreads), 0, s, a);
  }
  if constexpr (WHICH == kLaunchDq) {
    if (nqb == 0 || a.BH == 0) return hipSuccess;
    a.n_blk = static_cast<int>(nqb);
    hipLaunchKernelGGL((bwd_dq32_kernel<D, MASK, CAUSAL>), dim3(unsigned(nqb * a.BH)), dim3(kBThreads), 0, s, a);
  }
  return hipGetLastError();
}

template <int WHICH, int D>
hipError_t launch_type32(const BwdArgs& a, int mask_kind, bool causal, hipStream_t s) {
  switch (mask_kind) {
    case JVPATTN_MASK_NONE:
      return causal ? launch_tiles32<WHICH, D, JVPATTN_MASK_NONE, true>(a, s)
                    : launch_tiles32<WHICH, D, JVPATTN_MASK_NONE, false>(a, s);
    case JVPATTN_MASK_BOOL:
      return causal ? launch_tiles32<WHICH, D, JVPATTN_MASK_BOOL, true>(a, s)
                    : launch_tiles32<WHICH, D, JVPATTN_MASK_BOOL, false>(a, s);
    case JVPATTN_MASK_BITS:
      return causal ? launch_tiles32<WHICH, D, JVPATTN_MASK_BITS, true>(a, s)
                    : launch_tiles32<WHICH, D, JVPATTN_MASK_BITS, false>(a, s);
    case kMaskAddT:
      return causal ? launch_tiles32<WHICH, D, kMaskAddT, true>(a, s) : launch_tiles32<WHICH, D, kMaskAddT, false>(a, s);
    default:
      return causal ? launch_tiles32<WHICH, D, JVPATTN_MASK_ADDITIVE, true>(a, s)
                    : launch_tiles32<WHICH, D, JVPATTN_MASK_ADDITIVE, false>(a, s);
  }
}

template <int WHICH, int D>
hipError_t bwd_launch_part(const BwdArgs& a, int64_t rows_q, jvpattn_dtype dtype, int mask_kind, bool causal,
                           bool pow2, hipStream_t s) {
  if (dtype == JVPATTN_F32) {
    if constexpr (D == 64) {
      if constexpr (WHICH == kLaunchRows) {
        if (rows_q == 0) return hipSuccess;
        const int64_t nb = (rows_q * (D / 4) + kBThreads - 1) / kBThreads;   // d/4 lanes per row
        if (nb > INT32_MAX) return hipErrorInvalidValue;
        hipLaunchKernelGGL((bwd_rows32_kernel<D>), dim3(unsigned(nb)), dim3(kBThreads), 0, s, a, rows_q);
        return hipGetLastError();
      } else {
        return launch_type32<WHICH, D>(a, mask_kind, causal, s);
      }
    } else {
      return hipErrorInvalidValue;   // the validator admits float32 at d = 64 only
    }
  }
  if constexpr (WHICH == kLaunchRows) {   // built into the key side's object
    if (rows_q == 0) return hipSuccess;
    const int64_t nb = (rows_q * (D / 8) + kBThreads - 1) / kBThreads;   // d/8 lanes per row
    if (nb > INT32_MAX) return hipErrorInvalidValue;
    if (dtype == JVPATTN_BF16)
      hipLaunchKernelGGL((bwd_rows_kernel<BF16, D>), dim3(unsigned(nb)), dim3(kBThreads), 0, s, a, rows_q);
    else
      hipLaunchKernelGGL((bwd_rows_kernel<F16, D>), dim3(unsigned(nb)), dim3(kBThreads), 0, s, a, rows_q);
    return hipGetLastError();
  } else {
    return dtype == JVPATTN_BF16 ? launch_type<WHICH, BF16, D>(a, mask_kind, causal, pow2, s)
                                 : launch_type<WHICH, F16, D>(a, mask_kind, causal, pow2, s);
  }
}


}  // namespace jvpattn
