// Prefill grouped GEMMs on MFMA: each expert's rows (contiguous after grouping)
// against that expert's weights, one fetch of a weight tile serving every row of
// the workgroup's row tile.
//   gate/up: [rows_e x d] x [d x 2*f] on v_mfma_f32_16x16x32_f16, GeGLU in the
//            epilogue, H_e kept in fp32 [rows_e x f];
//   down:    [rows_e x f] x [f x d], fp32 output per (row, slot) pair.
//
// The 4-bit weights are not dequantised element by element. The affine form is
// factored out of the contraction per group of 64 columns:
//   sum_i (s q_i + b) a_i = s * sum_i q_i a_i + b * A_g,
// where A_g is the group sum of the activations; MFMA computes sum_i q_i a_i per
// group and the epilogue applies s and b. The B operand is the exact fp16 code q,
// made from one packed code word (see codes_f16), so the weights enter the
// product exactly; only the activations are rounded (to fp16, 11 bits):
// x from bf16 is exact, H from fp32 loses at most 2^-12 relative. Every
// activation row is scaled by a power of two so its largest magnitude lands in
// [2^14, 2^15) first (exact), and results are scaled back exactly.
//
// Each wavefront loads its own weight fragments straight from the packed tiles
// (the tile layout gives lane l the code word of row l%16, columns 8*(l/16)..+7)
// with kRing groups in flight; activation tiles are staged once per group in
// double-buffered LDS and shared by the workgroup's four waves.
#pragma once

#include "common.h"

namespace qmoe {

constexpr int kLdsStride = 72;  // halfs per LDS row: 64 + 8 padding (144 B) against bank conflicts
constexpr int kRing = 4;        // weight groups in flight per wavefront
constexpr int kMaxGroups = 96;  // d_model or d_ff up to 6144

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

struct PrefillArgs {
  const uint8_t* pool;
  uint64_t stride, n_blobs;
  const uint32_t* slot_table;
  const uint8_t* shared_blob;
  const int32_t* offset;  // [E+1] sorted-pair ranges per expert (routed)
  const int32_t* perm;    // [rows*top_k]
  int d, f, fs, n_experts, top_k, rows;
  int routed_mtiles;      // upper bound of routed 64-row tiles
  int shared_mtiles;      // 64-row tiles of the shared expert
  float* xscale;          // [rows] power-of-two activation scale per row
  uint16_t* xh;           // [rows][d] fp16 of x * scale
  uint16_t* xl;           // [rows][d] fp16 remainder (fp32 x only)
  float* xg;              // [rows][d/64] group sums of the scaled fp16 activations (hi + lo)
  float* H;               // routed GeGLU output, fp32 [rows*top_k][f] (sorted-pair order)
  float* Hs;              // shared GeGLU output, fp32 [rows][fs]
  float* hg;              // routed H group sums [rows*top_k][f/64], then shared [rows][fs/64]
  uint32_t* hmax;         // [rows*top_k] max |H| per routed row (float bits), then [rows] shared
  float* expert_out;      // [rows*top_k][d]
  float* shared_out;      // [rows][d]
};

// 64-row tile -> (expert, first sorted position, row count); expert -1 = shared
struct MTile {
  int e, m0, mrows;
  const uint8_t* blob;
  int F;
};

// Routed tiles are numbered expert by expert (ceil(count_e / 64) tiles each).
// The wavefront finds tile `mt` with a prefix sum over the per-expert tile counts
// (lane l covers experts [l*epl, (l+1)*epl)). Every lane returns the same tile.
__device__ __forceinline__ bool find_mtile(const PrefillArgs& A, bool shared, int mt, MTile& T) {
  if (shared) {
    if (mt >= A.shared_mtiles) return false;
    T.e = -1;
    T.m0 = 64 * mt;
    T.mrows = min(64, A.rows - T.m0);
    T.blob = A.shared_blob;
    T.F = A.fs;
    return true;
  }
  if (mt >= A.routed_mtiles) return false;
  const int lane = threadIdx.x & 63;
  const int epl = A.n_experts / 64;
  int mine = 0;
  for (int j = 0; j < epl; ++j) {
    const int e = lane * epl + j;
    mine += (A.offset[e + 1] - A.offset[e] + 63) >> 6;
  }
  int incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  const int excl = incl - mine;
  const uint64_t hit = __ballot(mt >= excl && mt < incl);
  if (hit == 0) return false;
  const int owner = __ffsll((unsigned long long)hit) - 1;
  int t = __shfl(excl, owner, 64);
  int e = owner * epl;
  for (;; ++e) {
    const int c = A.offset[e + 1] - A.offset[e];
    const int nt = (c + 63) >> 6;
    if (mt < t + nt) {
      T.e = e;
      T.m0 = A.offset[e] + 64 * (mt - t);
      T.mrows = min(64, c - 64 * (mt - t));
      T.F = A.f;
      T.blob = expert_blob(A.pool, A.stride, A.n_blobs, A.slot_table, e, A.n_experts);
      return T.blob != nullptr;
    }
    t += nt;
  }
}

// power of two that brings a row maximum m (> 0) into [2^14, 2^15); 1 for m == 0
__device__ __forceinline__ float row_scale(float m) {
  if (!(m > 0.0f)) return 1.0f;
  const int e = (int)((__float_as_uint(m) >> 23) & 0xff) - 127;  // floor(log2 m) for normal m
  return ldexpf(1.0f, min(14 - e, 126));
}

__device__ __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ uint16_t f16_bits(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }
__device__ __forceinline__ float f16_val(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// B operand: the 8 codes of one packed word as exact fp16 values q (0..15): the
// pair (1024 + q, 1024 + q') is built with a mask and an OR of the exponent of
// 1024 (0x6400), then 1024 is subtracted with one packed fp16 add per pair.
__device__ __forceinline__ f16x8_t codes_f16(uint32_t w) {
  const f16x2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  f16x2_t p[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    p[t] = __builtin_bit_cast(f16x2_t, ((w >> (4 * t)) & 0x000F000Fu) | 0x64006400u) - k1024;
  return f16x8_t{p[0].x, p[0].y, p[1].x, p[1].y, p[2].x, p[2].y, p[3].x, p[3].y};
}

__device__ __forceinline__ f16x8_t lds_frag(const uint16_t* p) {
  return __builtin_bit_cast(f16x8_t, *reinterpret_cast<const uint4*>(p));
}

// ---------------------------------------------------------------- activation pre-pass

// One workgroup per activation row: power-of-two scale, fp16 copy (x * scale, plus
// the fp16 rounding remainder for fp32 x), group sums of the fp16 values, and the
// clearing of the row's H maxima (its routed pairs, then its shared-expert row).
template <typename XT>
__global__ __launch_bounds__(256) void k_prefill_prep(const XT* __restrict__ x, int rows, int d, int top_k,
                                                      float* __restrict__ xscale, uint16_t* __restrict__ xh,
                                                      uint16_t* __restrict__ xl, float* __restrict__ xg,
                                                      uint32_t* __restrict__ hmax) {
  constexpr bool kLo = sizeof(XT) == 4;
  __shared__ float red[4];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const XT* xr = x + (size_t)r * d;
  float m = 0.0f;
  for (int i = tid; i < d; i += 256) m = fmaxf(m, fabsf(to_f32(xr[i])));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  const float sc = row_scale(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
  if (tid == 0) xscale[r] = sc;
  if (tid < top_k) hmax[r * top_k + tid] = 0u;
  if (tid == 0) hmax[rows * top_k + r] = 0u;
  const int G = d / kGroup;
  for (int g = wave; g < G; g += 4) {
    const int i = g * kGroup + lane;
    const float v = to_f32(xr[i]) * sc;
    const uint16_t hb = f16_bits(v);
    float s = f16_val(hb);
    xh[(size_t)r * d + i] = hb;
    if (kLo) {
      const uint16_t lb = f16_bits(v - f16_val(hb));
      xl[(size_t)r * d + i] = lb;
      s += f16_val(lb);
    }
    s = wave_sum(s);
    if (lane == 0) xg[(size_t)r * G + g] = s;
  }
}

// ---------------------------------------------------------------- shared GEMM core

// Accumulates a [64-row tile] x [one 16-column n-block per matrix, NM matrices] product
// over K groups: acc[mb][m] += s * sum q a + b * a_g, per group.
// A (activations, fp16, row-scaled) arrives through LDS; `stage(g, buf)` must fill
// LDS buffer `buf` with group g. B comes from the packed tiles at wbase[m] +
// g * kTile4 (+ kh*1024 + row*16 + (lane/16)*4), scales at + 2048 + row*4.
template <int NM, bool LO>
struct GemmCore {
  f32x4_t acc[4][NM];
  uint32_t cw[kRing][NM][2];
  uint32_t sb[kRing][NM];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[i][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  __device__ __forceinline__ void load_b(int slot, const uint8_t* const* wbase, int g, int row, int lane) {
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const uint8_t* t = wbase[m] + (uint64_t)g * kTile4;
      cw[slot][m][0] = ldg4(t + row * 16 + (lane >> 4) * 4);
      cw[slot][m][1] = ldg4(t + 1024 + row * 16 + (lane >> 4) * 4);
      sb[slot][m] = ldg4(t + kTile4Codes + row * 4);
    }
  }
};

// ---------------------------------------------------------------- gate/up + GeGLU

// Workgroup = (64-row tile, 64 d_ff columns). Wave w owns d_ff columns [16w, +16) of
// both gate and up (so GeGLU runs in registers) for every row of the tile.
// Routed tiles first: blockIdx < routed_mtiles * f/64, then shared tiles.
template <bool LO>
__global__ __launch_bounds__(256) void k_prefill_gateup(PrefillArgs A) {
  __shared__ __attribute__((aligned(16))) uint16_t Xs[2][64 * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t Xls[LO ? 2 : 1][LO ? 64 * kLdsStride : 8];
  extern __shared__ float4 dyn_lds[];  // [G][64] activation group sums
  float(*XgL)[64] = reinterpret_cast<float(*)[64]>(dyn_lds);
  __shared__ int rowsrc[64];
  __shared__ float rowinv[64];
  __shared__ float hsumL[4][64];

  const int nfr = A.f / 64;
  int b = blockIdx.x;
  bool shared = false;
  int nfc = nfr;
  if (b >= A.routed_mtiles * nfr) {
    b -= A.routed_mtiles * nfr;
    shared = true;
    nfc = A.fs / 64;
  }
  const int mt = b / nfc, fc = b % nfc;
  MTile T;
  if (!find_mtile(A, shared, mt, T)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = A.d / kGroup;
  const int nmb = (T.mrows + 15) >> 4;

  if (tid < 64) {
    int src = -1;
    if (tid < T.mrows) src = (T.e >= 0) ? A.perm[T.m0 + tid] / A.top_k : T.m0 + tid;
    rowsrc[tid] = src;
    rowinv[tid] = src >= 0 ? 1.0f / A.xscale[src] : 1.0f;  // exact: a power of two
  }
  __syncthreads();
  for (int i = tid; i < 64 * G; i += 256) {
    const int r = i / G, g = i % G;
    const int src = rowsrc[r];
    XgL[g][r] = src >= 0 ? A.xg[(size_t)src * G + g] : 0.0f;
  }

  // this wave's weight rows: row 16*wave + lane%16 of the 64-row block fc of gate and up
  const int wrow = 16 * wave + (lane & 15);
  const uint8_t* wbase[2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
    wbase[m] = T.blob + (uint64_t)m * m4_bytes(T.F, A.d) + (uint64_t)fc * G * kTile4;
  GemmCore<2, LO> C;
  C.zero();
#pragma unroll
  for (int j = 0; j < kRing; ++j)
    if (j < G) C.load_b(j, wbase, j, wrow, lane);

  // activation staging: thread -> row tid/4, 16 halfs at column (tid%4)*16
  const int xr = tid >> 2, xq = tid & 3;
  const int xsrc = rowsrc[xr];
  const uint16_t* xrow = A.xh + (size_t)(xsrc >= 0 ? xsrc : 0) * A.d + xq * 16;
  const uint16_t* xrowl = LO ? A.xl + (size_t)(xsrc >= 0 ? xsrc : 0) * A.d + xq * 16 : nullptr;
  uint4 xa[2], xla[2];
  auto xload = [&](int g) {
    if (xsrc >= 0) {
      xa[0] = *reinterpret_cast<const uint4*>(xrow + g * kGroup);
      xa[1] = *reinterpret_cast<const uint4*>(xrow + g * kGroup + 8);
      if (LO) {
        xla[0] = *reinterpret_cast<const uint4*>(xrowl + g * kGroup);
        xla[1] = *reinterpret_cast<const uint4*>(xrowl + g * kGroup + 8);
      }
    } else {
      xa[0] = xa[1] = xla[0] = xla[1] = make_uint4(0, 0, 0, 0);
    }
  };
  auto xstore = [&](int buf) {
    uint4* d = reinterpret_cast<uint4*>(&Xs[buf][xr * kLdsStride + xq * 16]);
    d[0] = xa[0];
    d[1] = xa[1];
    if (LO) {
      uint4* dl = reinterpret_cast<uint4*>(&Xls[buf][xr * kLdsStride + xq * 16]);
      dl[0] = xla[0];
      dl[1] = xla[1];
    }
  };
  xload(0);
  xstore(0);
  if (G > 1) xload(1);
  __syncthreads();

  for (int g0 = 0; g0 < G; g0 += kRing) {
#pragma unroll
    for (int j = 0; j < kRing; ++j) {
      const int g = g0 + j;
      if (g < G) {
        const int buf = g & 1;
        // B fragments and scales of this group, then refill the ring slot
        f16x8_t bfr[2][2];
        float s[2], bp[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          bfr[m][0] = codes_f16(C.cw[j][m][0]);
          bfr[m][1] = codes_f16(C.cw[j][m][1]);
          s[m] = bf16_lo(C.sb[j][m]);
          bp[m] = bf16_hi(C.sb[j][m]);
        }
        if (g + kRing < G) C.load_b(j, wbase, g + kRing, wrow, lane);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          if (mb < nmb) {
            const int arow = 16 * mb + (lane & 15);
            const f16x8_t a0 = lds_frag(&Xs[buf][arow * kLdsStride + 8 * (lane >> 4)]);
            const f16x8_t a1 = lds_frag(&Xs[buf][arow * kLdsStride + 32 + 8 * (lane >> 4)]);
            const float4 xg4 = *reinterpret_cast<const float4*>(&XgL[g][16 * mb + 4 * (lane >> 4)]);
            const float xgv[4] = {xg4.x, xg4.y, xg4.z, xg4.w};
#pragma unroll
            for (int m = 0; m < 2; ++m) {
              f32x4_t t = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bfr[m][0], f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
              t = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bfr[m][1], t, 0, 0, 0);
              if (LO) {
                const f16x8_t l0 = lds_frag(&Xls[buf][arow * kLdsStride + 8 * (lane >> 4)]);
                const f16x8_t l1 = lds_frag(&Xls[buf][arow * kLdsStride + 32 + 8 * (lane >> 4)]);
                t = __builtin_amdgcn_mfma_f32_16x16x32_f16(l0, bfr[m][0], t, 0, 0, 0);
                t = __builtin_amdgcn_mfma_f32_16x16x32_f16(l1, bfr[m][1], t, 0, 0, 0);
              }
#pragma unroll
              for (int i = 0; i < 4; ++i) C.acc[mb][m][i] = fmaf(s[m], t[i], fmaf(bp[m], xgv[i], C.acc[mb][m][i]));
            }
          }
        }
        // next activation group into the other buffer (its readers passed the last barrier)
        if (g + 1 < G) xstore(buf ^ 1);
        if (g + 2 < G) xload(g + 2);
        __syncthreads();
      }
    }
  }

  // GeGLU epilogue: lane holds rows 16mb + 4*(lane/16) + i, d_ff column fc*64 + 16*wave + lane%16
  float* H = (T.e >= 0) ? A.H : A.Hs;
  float* hg = (T.e >= 0) ? A.hg : A.hg + (size_t)A.rows * A.top_k * (A.f / 64);
  uint32_t* hmax = (T.e >= 0) ? A.hmax : A.hmax + (size_t)A.rows * A.top_k;
  const int F = T.F, nG = F / 64;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * mb + 4 * (lane >> 4) + i;
      float h = 0.0f;
      if (r < T.mrows) {
        const float inv = rowinv[r];
        h = gelu_tanh(C.acc[mb][0][i] * inv) * (C.acc[mb][1][i] * inv);
        H[(size_t)(T.m0 + r) * F + fc * 64 + 16 * wave + (lane & 15)] = h;
      }
      // over the 16 lanes holding this row: max |h| (row scale of the down GEMM) and sum
      float mx = fabsf(h), sm = h;
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) {
        mx = fmaxf(mx, __shfl_xor(mx, off, 64));
        sm += __shfl_xor(sm, off, 64);
      }
      if ((lane & 15) == 0 && r < 64) {
        if (r < T.mrows) atomicMax(&hmax[T.m0 + r], __float_as_uint(mx));
        hsumL[wave][r] = sm;
      }
    }
  __syncthreads();
  if (tid < T.mrows)
    hg[(size_t)(T.m0 + tid) * nG + fc] = ((hsumL[0][tid] + hsumL[1][tid]) + hsumL[2][tid]) + hsumL[3][tid];
}

// ---------------------------------------------------------------- down

// Workgroup = (64-row tile, 64 output columns). Wave w owns output columns [16w, +16)
// for every row of the tile. Routed tiles first, then shared.
__global__ __launch_bounds__(256) void k_prefill_down(PrefillArgs A) {
  __shared__ __attribute__((aligned(16))) uint16_t Hl[2][64 * kLdsStride];
  __shared__ float rowsc[64];
  extern __shared__ float4 dyn_lds[];  // [G][64] H group sums (scaled)
  float(*hgL)[64] = reinterpret_cast<float(*)[64]>(dyn_lds);
  const int NBd = A.d / 64;
  int b = blockIdx.x;
  bool shared = false;
  if (b >= A.routed_mtiles * NBd) {
    b -= A.routed_mtiles * NBd;
    shared = true;
  }
  const int mt = b / NBd, nb = b % NBd;
  MTile T;
  if (!find_mtile(A, shared, mt, T)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int F = T.F, G = F / kGroup;
  const int nmb = (T.mrows + 15) >> 4;
  const float* Hsrc = (T.e >= 0) ? A.H : A.Hs;
  const float* hg = (T.e >= 0) ? A.hg : A.hg + (size_t)A.rows * A.top_k * (A.f / 64);
  const uint32_t* hmax = (T.e >= 0) ? A.hmax : A.hmax + (size_t)A.rows * A.top_k;
  if (tid < 64) rowsc[tid] = tid < T.mrows ? row_scale(__uint_as_float(hmax[T.m0 + tid])) : 1.0f;
  __syncthreads();
  for (int i = tid; i < 64 * G; i += 256) {
    const int r = i / G, g = i % G;
    hgL[g][r] = r < T.mrows ? hg[(size_t)(T.m0 + r) * G + g] * rowsc[r] : 0.0f;
  }

  const int wrow = 16 * wave + (lane & 15);
  const uint8_t* wbase[1] = {T.blob + 2 * m4_bytes(F, A.d) + (uint64_t)nb * G * kTile4};
  GemmCore<1, false> C;
  C.zero();
#pragma unroll
  for (int j = 0; j < kRing; ++j)
    if (j < G) C.load_b(j, wbase, j, wrow, lane);

  // H staging: thread -> row tid/4, 16 values at column (tid%4)*16, scaled to fp16
  const int hr = tid >> 2, hq = tid & 3;
  const bool hvalid = hr < T.mrows;
  const float hsc = rowsc[hr];
  const float* hrow = Hsrc + (size_t)(T.m0 + (hvalid ? hr : 0)) * F + hq * 16;
  float4 hv[4];
  auto hload = [&](int g) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      hv[i] = hvalid ? *reinterpret_cast<const float4*>(hrow + g * kGroup + 4 * i) : make_float4(0.f, 0.f, 0.f, 0.f);
  };
  auto hstore = [&](int buf) {
    uint32_t p[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[2 * i] = (uint32_t)f16_bits(hv[i].x * hsc) | ((uint32_t)f16_bits(hv[i].y * hsc) << 16);
      p[2 * i + 1] = (uint32_t)f16_bits(hv[i].z * hsc) | ((uint32_t)f16_bits(hv[i].w * hsc) << 16);
    }
    uint4* d = reinterpret_cast<uint4*>(&Hl[buf][hr * kLdsStride + hq * 16]);
    d[0] = make_uint4(p[0], p[1], p[2], p[3]);
    d[1] = make_uint4(p[4], p[5], p[6], p[7]);
  };
  hload(0);
  hstore(0);
  if (G > 1) hload(1);
  __syncthreads();

  for (int g0 = 0; g0 < G; g0 += kRing) {
#pragma unroll
    for (int j = 0; j < kRing; ++j) {
      const int g = g0 + j;
      if (g < G) {
        const int buf = g & 1;
        const f16x8_t b0 = codes_f16(C.cw[j][0][0]);
        const f16x8_t b1 = codes_f16(C.cw[j][0][1]);
        const float s = bf16_lo(C.sb[j][0]);
        const float bp = bf16_hi(C.sb[j][0]);
        if (g + kRing < G) C.load_b(j, wbase, g + kRing, wrow, lane);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          if (mb < nmb) {
            const int arow = 16 * mb + (lane & 15);
            const f16x8_t a0 = lds_frag(&Hl[buf][arow * kLdsStride + 8 * (lane >> 4)]);
            const f16x8_t a1 = lds_frag(&Hl[buf][arow * kLdsStride + 32 + 8 * (lane >> 4)]);
            const float4 hg4 = *reinterpret_cast<const float4*>(&hgL[g][16 * mb + 4 * (lane >> 4)]);
            const float hgv[4] = {hg4.x, hg4.y, hg4.z, hg4.w};
            f32x4_t t = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b0, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b1, t, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) C.acc[mb][0][i] = fmaf(s, t[i], fmaf(bp, hgv[i], C.acc[mb][0][i]));
          }
        }
        if (g + 1 < G) hstore(buf ^ 1);
        if (g + 2 < G) hload(g + 2);
        __syncthreads();
      }
    }
  }
  float* out = (T.e >= 0) ? A.expert_out : A.shared_out;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * mb + 4 * (lane >> 4) + i;
      if (r < T.mrows) out[(size_t)(T.m0 + r) * A.d + nb * 64 + 16 * wave + (lane & 15)] = C.acc[mb][0][i] / rowsc[r];
    }
}

}  // namespace qmoe
