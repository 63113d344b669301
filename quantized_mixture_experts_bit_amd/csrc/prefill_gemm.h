// Prefill grouped GEMMs on MFMA: each expert's rows (contiguous after grouping)
// against that expert's weights, one fetch of a weight tile serving every row of
// the workgroup's row tile.
//   gate/up: [rows_e x d] x [d x 2*f] on v_mfma_f32_16x16x32_f16, GeGLU in the
//            epilogue, H_e kept in fp32 [rows_e x f];
//   down:    [rows_e x f] x [f x d], fp32 output per (row, slot) pair.
//
// Operands are fp16 (11 significant bits): the dequantised weight s*q + b is
// rounded once to fp16 (fp32 fma, RNE), bf16 activations convert exactly, and
// the fp32 GeGLU output H is rounded to fp16. Rounding to bf16 instead (8 bits)
// costs up to 5e-3 of ||y||_inf on these shapes; fp16 keeps it near 5e-4 at the
// same MFMA rate. Range: every activation row is scaled by a power of two so its
// largest magnitude lands in [2^14, 2^15) before the conversion (exact), and
// the fp32 accumulators are scaled back exactly.
//
// The K loop keeps kRing groups of weights and activations in flight per thread
// (a register ring), so each workgroup overlaps HBM latency with its MFMAs.
#pragma once

#include "common.h"

namespace qmoe {

constexpr int kLdsStride = 72;  // halfs per LDS row: 64 + 8 padding (144 B) against bank conflicts
constexpr int kRing = 4;        // groups in flight per thread

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
  const float* xscale;    // [rows] power-of-two activation scale per row
  float* H;               // routed GeGLU output, fp32 [rows*top_k][f] (sorted-pair order)
  float* Hs;              // shared GeGLU output, fp32 [rows][fs]
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

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const _Float16 ha = (_Float16)a, hb = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// power of two that brings a row maximum m (> 0) into [2^14, 2^15); 1 for m == 0
__device__ __forceinline__ float row_scale(float m) {
  if (!(m > 0.0f)) return 1.0f;
  const int e = (int)((__float_as_uint(m) >> 23) & 0xff) - 127;  // floor(log2 m) for normal m
  return ldexpf(1.0f, min(14 - e, 126));
}

// Dequantise 16 consecutive columns (two code words) of one row to fp16 and store
// them to LDS row `dst_row` at column `col0` (w = s*q + b in fp32, RNE to fp16).
__device__ __forceinline__ void dequant16_to_lds(uint2 cw, uint32_t sbw, uint16_t* dst_row, int col0) {
  const float s = bf16_lo(sbw), b = bf16_hi(sbw);
  const uint32_t ws[2] = {cw.x, cw.y};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    uint32_t out[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float q0 = (float)((ws[i] >> (4 * t)) & 0xFu);
      const float q1 = (float)((ws[i] >> (16 + 4 * t)) & 0xFu);
      out[t] = pack_f16x2(fmaf(s, q0, b), fmaf(s, q1, b));
    }
    *reinterpret_cast<uint4*>(dst_row + col0 + 8 * i) = make_uint4(out[0], out[1], out[2], out[3]);
  }
}

__device__ __forceinline__ f16x8_t lds_frag(const uint16_t* p) {
  return __builtin_bit_cast(f16x8_t, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ void zero16(uint16_t* p) {
  reinterpret_cast<uint4*>(p)[0] = make_uint4(0, 0, 0, 0);
  reinterpret_cast<uint4*>(p)[1] = make_uint4(0, 0, 0, 0);
}

// 16 consecutive activation values held in registers between load and staging
template <typename T>
struct Piece16;
template <>
struct Piece16<uint16_t> {  // bf16
  uint4 v[2];
  __device__ __forceinline__ void load(const uint16_t* p) {
    v[0] = reinterpret_cast<const uint4*>(p)[0];
    v[1] = reinterpret_cast<const uint4*>(p)[1];
  }
  __device__ __forceinline__ float get(int i) const {
    const uint32_t w = reinterpret_cast<const uint32_t*>(v)[i >> 1];
    return (i & 1) ? bf16_hi(w) : bf16_lo(w);
  }
};
template <>
struct Piece16<float> {
  uint4 v[4];
  __device__ __forceinline__ void load(const float* p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = reinterpret_cast<const uint4*>(p)[i];
  }
  __device__ __forceinline__ float get(int i) const { return __uint_as_float(reinterpret_cast<const uint32_t*>(v)[i]); }
};

// store 16 values times a power-of-two scale as fp16 hi (+ lo = rounding remainder)
template <typename T, bool LO>
__device__ __forceinline__ void stage16(const Piece16<T>& pc, float sc, uint16_t* hi, uint16_t* lo) {
  uint32_t h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = pc.get(2 * i) * sc, b = pc.get(2 * i + 1) * sc;
    const _Float16 ha = (_Float16)a, hb = (_Float16)b;
    h[i] = (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
    if (LO) l[i] = pack_f16x2(a - (float)ha, b - (float)hb);
  }
  reinterpret_cast<uint4*>(hi)[0] = make_uint4(h[0], h[1], h[2], h[3]);
  reinterpret_cast<uint4*>(hi)[1] = make_uint4(h[4], h[5], h[6], h[7]);
  if (LO) {
    reinterpret_cast<uint4*>(lo)[0] = make_uint4(l[0], l[1], l[2], l[3]);
    reinterpret_cast<uint4*>(lo)[1] = make_uint4(l[4], l[5], l[6], l[7]);
  }
}

__device__ __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }
__device__ __forceinline__ float to_f32(float v) { return v; }

// ---------------------------------------------------------------- scales pre-pass

// One workgroup per activation row: its power-of-two scale; also clears the
// H row maxima of the row's routed pairs and of its shared-expert row.
template <typename XT>
__global__ __launch_bounds__(256) void k_prefill_scales(const XT* __restrict__ x, int rows, int d, int top_k,
                                                        float* __restrict__ xscale, uint32_t* __restrict__ hmax) {
  __shared__ float red[4];
  const int r = blockIdx.x;
  float m = 0.0f;
  for (int i = threadIdx.x; i < d; i += 256) m = fmaxf(m, fabsf(to_f32(x[(size_t)r * d + i])));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) xscale[r] = row_scale(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
  if (threadIdx.x < top_k) hmax[r * top_k + threadIdx.x] = 0u;
  if (threadIdx.x == 0) hmax[rows * top_k + r] = 0u;
}

// ---------------------------------------------------------------- gate/up + GeGLU

// Workgroup = (64-row tile, 32 d_ff columns). 4 waves: wave (wm, wn) owns rows
// [32 wm, +32) and d_ff columns [16 wn, +16) of both gate and up, so GeGLU is
// applied in registers. grid.x = mtiles * F/32 (routed or shared launch).
template <typename XT>
__global__ __launch_bounds__(256) void k_prefill_gateup(PrefillArgs A, const XT* __restrict__ x, int shared) {
  constexpr bool kLo = sizeof(XT) == 4;
  __shared__ __attribute__((aligned(16))) uint16_t Xh[64 * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t Xl[kLo ? 64 * kLdsStride : 8];
  __shared__ __attribute__((aligned(16))) uint16_t W[2][32 * kLdsStride];
  __shared__ int rowsrc[64];
  __shared__ float rowsc[64];

  const int nfc = (shared ? A.fs : A.f) / 32;
  const int mt = blockIdx.x / nfc;
  const int fc = blockIdx.x % nfc;
  MTile T;
  if (!find_mtile(A, shared != 0, mt, T)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int G = A.d / kGroup;

  if (tid < 64) {
    int src = -1;
    if (tid < T.mrows) src = (T.e >= 0) ? A.perm[T.m0 + tid] / A.top_k : T.m0 + tid;
    rowsrc[tid] = src;
    rowsc[tid] = src >= 0 ? A.xscale[src] : 1.0f;
  }
  __syncthreads();

  // weight piece this thread dequantises: matrix wmat, row wr of the 32, 16 columns
  const int wmat = tid >> 7;
  const int wr = (tid & 127) >> 2;
  const int piece = tid & 3;  // half = piece >> 1, words (piece & 1) * 2 .. +1
  const int wh = piece >> 1, wj = (piece & 1) * 2;
  const int f0 = fc * 32;
  const int trow = (f0 & 63) + wr;  // row inside the 64-row tile
  const uint8_t* wbase = T.blob + (uint64_t)wmat * m4_bytes(T.F, A.d) + (uint64_t)(f0 >> 6) * G * kTile4 +
                         wh * 1024 + trow * 16 + wj * 4;
  const uint8_t* sbase = T.blob + (uint64_t)wmat * m4_bytes(T.F, A.d) + (uint64_t)(f0 >> 6) * G * kTile4 +
                         kTile4Codes + trow * 4;
  // activation piece: row xr, 16 columns
  const int xr = tid >> 2, xq = tid & 3;
  const int xsrc = rowsrc[xr];
  const float xsc = rowsc[xr];
  const XT* xrow = x + (size_t)(xsrc >= 0 ? xsrc : 0) * A.d + xq * 16;

  uint2 cw[kRing];
  uint32_t sb[kRing];
  Piece16<XT> xp[kRing];
#pragma unroll
  for (int j = 0; j < kRing; ++j) {
    if (j < G) {
      cw[j] = *reinterpret_cast<const uint2*>(wbase + (uint64_t)j * kTile4);
      sb[j] = ldg4(sbase + (uint64_t)j * kTile4);
      if (xsrc >= 0) xp[j].load(xrow + j * kGroup);
    }
  }

  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int g0 = 0; g0 < G; g0 += kRing) {
#pragma unroll
    for (int j = 0; j < kRing; ++j) {
      const int g = g0 + j;
      if (g < G) {
        dequant16_to_lds(cw[j], sb[j], &W[wmat][wr * kLdsStride], wh * 32 + wj * 8);
        uint16_t* hi = &Xh[xr * kLdsStride + xq * 16];
        uint16_t* lo = kLo ? &Xl[xr * kLdsStride + xq * 16] : nullptr;
        if (xsrc >= 0) {
          stage16<XT, kLo>(xp[j], xsc, hi, lo);
        } else {
          zero16(hi);
          if (kLo) zero16(lo);
        }
        __syncthreads();
        if (g + kRing < G) {  // refill this ring slot while the MFMAs run
          cw[j] = *reinterpret_cast<const uint2*>(wbase + (uint64_t)(g + kRing) * kTile4);
          sb[j] = ldg4(sbase + (uint64_t)(g + kRing) * kTile4);
          if (xsrc >= 0) xp[j].load(xrow + (g + kRing) * kGroup);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int kc = kk * 32 + 8 * (lane >> 4);
          f16x8_t bfr[2];
#pragma unroll
          for (int m = 0; m < 2; ++m) bfr[m] = lds_frag(&W[m][(16 * wn + (lane & 15)) * kLdsStride + kc]);
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            const int row = 32 * wm + 16 * mb + (lane & 15);
            const f16x8_t afr = lds_frag(&Xh[row * kLdsStride + kc]);
#pragma unroll
            for (int m = 0; m < 2; ++m)
              acc[mb][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr, bfr[m], acc[mb][m], 0, 0, 0);
            if (kLo) {
              const f16x8_t alo = lds_frag(&Xl[row * kLdsStride + kc]);
#pragma unroll
              for (int m = 0; m < 2; ++m)
                acc[mb][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bfr[m], acc[mb][m], 0, 0, 0);
            }
          }
        }
        __syncthreads();
      }
    }
  }
  // GeGLU epilogue: lane holds rows 4*(lane/16) + i of each 16-row block, column lane % 16
  float* H = (T.e >= 0) ? A.H : A.Hs;
  uint32_t* hmax = (T.e >= 0) ? A.hmax : A.hmax + (size_t)A.rows * A.top_k;
  const int F = T.F;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 32 * wm + 16 * mb + 4 * (lane >> 4) + i;
      const float inv = 1.0f / rowsc[r];  // exact: a power of two
      float h = 0.0f;
      if (r < T.mrows) {
        h = gelu_tanh(acc[mb][0][i] * inv) * (acc[mb][1][i] * inv);
        H[(size_t)(T.m0 + r) * F + f0 + 16 * wn + (lane & 15)] = h;
      }
      // row maximum over the 16 lanes holding this row, one atomic per row and wave
      float m = fabsf(h);
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
      if ((lane & 15) == 0 && r < T.mrows) atomicMax(&hmax[T.m0 + r], __float_as_uint(m));
    }
}

// ---------------------------------------------------------------- down

// Workgroup = (64-row tile, 64 output columns). 4 waves: wave (wm, wn) owns rows
// [32 wm, +32) and columns [32 wn, +32). grid.x = mtiles * d/64.
__global__ __launch_bounds__(256) void k_prefill_down(PrefillArgs A, int shared) {
  __shared__ __attribute__((aligned(16))) uint16_t Hl[64 * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t W[64 * kLdsStride];
  __shared__ float rowsc[64];
  const int NBd = A.d / 64;
  const int mt = blockIdx.x / NBd;
  const int nb = blockIdx.x % NBd;
  MTile T;
  if (!find_mtile(A, shared != 0, mt, T)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int F = T.F, G = F / kGroup;
  const float* Hsrc = (T.e >= 0) ? A.H : A.Hs;
  const uint32_t* hmax = (T.e >= 0) ? A.hmax : A.hmax + (size_t)A.rows * A.top_k;
  const int wr = tid >> 2, piece = tid & 3;
  const int wh = piece >> 1, wj = (piece & 1) * 2;
  const uint8_t* tile0 = T.blob + 2 * m4_bytes(F, A.d) + (uint64_t)nb * G * kTile4;
  const uint8_t* wbase = tile0 + wh * 1024 + wr * 16 + wj * 4;
  const uint8_t* sbase = tile0 + kTile4Codes + wr * 4;
  const int hr = tid >> 2, hq = tid & 3;
  if (tid < 64) rowsc[tid] = tid < T.mrows ? row_scale(__uint_as_float(hmax[T.m0 + tid])) : 1.0f;
  __syncthreads();
  const float hsc = rowsc[hr];
  const bool hvalid = hr < T.mrows;
  const float* hrow = Hsrc + (size_t)(T.m0 + (hvalid ? hr : 0)) * F + hq * 16;

  uint2 cw[kRing];
  uint32_t sb[kRing];
  Piece16<float> hp[kRing];
#pragma unroll
  for (int j = 0; j < kRing; ++j) {
    if (j < G) {
      cw[j] = *reinterpret_cast<const uint2*>(wbase + (uint64_t)j * kTile4);
      sb[j] = ldg4(sbase + (uint64_t)j * kTile4);
      if (hvalid) hp[j].load(hrow + j * kGroup);
    }
  }

  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int g0 = 0; g0 < G; g0 += kRing) {
#pragma unroll
    for (int j = 0; j < kRing; ++j) {
      const int g = g0 + j;
      if (g < G) {
        dequant16_to_lds(cw[j], sb[j], &W[wr * kLdsStride], wh * 32 + wj * 8);
        uint16_t* dst = &Hl[hr * kLdsStride + hq * 16];
        if (hvalid)
          stage16<float, false>(hp[j], hsc, dst, nullptr);
        else
          zero16(dst);
        __syncthreads();
        if (g + kRing < G) {
          cw[j] = *reinterpret_cast<const uint2*>(wbase + (uint64_t)(g + kRing) * kTile4);
          sb[j] = ldg4(sbase + (uint64_t)(g + kRing) * kTile4);
          if (hvalid) hp[j].load(hrow + (g + kRing) * kGroup);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int kc = kk * 32 + 8 * (lane >> 4);
          f16x8_t bfr[2];
#pragma unroll
          for (int nbk = 0; nbk < 2; ++nbk)
            bfr[nbk] = lds_frag(&W[(32 * wn + 16 * nbk + (lane & 15)) * kLdsStride + kc]);
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            const f16x8_t afr = lds_frag(&Hl[(32 * wm + 16 * mb + (lane & 15)) * kLdsStride + kc]);
#pragma unroll
            for (int nbk = 0; nbk < 2; ++nbk)
              acc[mb][nbk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr, bfr[nbk], acc[mb][nbk], 0, 0, 0);
          }
        }
        __syncthreads();
      }
    }
  }
  float* out = (T.e >= 0) ? A.expert_out : A.shared_out;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nbk = 0; nbk < 2; ++nbk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 32 * wm + 16 * mb + 4 * (lane >> 4) + i;
        if (r < T.mrows)
          out[(size_t)(T.m0 + r) * A.d + nb * 64 + 32 * wn + 16 * nbk + (lane & 15)] = acc[mb][nbk][i] / rowsc[r];
      }
}

}  // namespace qmoe
