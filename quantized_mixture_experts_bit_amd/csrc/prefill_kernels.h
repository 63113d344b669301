// Prefill chunk: token->expert grouping and grouped GEMMs on MFMA.
//
// Prefill works on chunks of rows so that one fetched expert serves every row of
// the chunk routed to it (blog-mushroom article "TurboFieldfare: Gemma 4 26B on
// an 8 GB MacBook", section "Why 26B Fits in 2 GB"; paperfeed digest
// "drumih/turbo-fieldfare", "How it works"). Here the (row, slot) pairs are
// grouped by expert with a stable counting sort, and each expert's rows run as
// one GEMM against that expert's weights:
//   gate/up: [rows_e x d] x [d x 2*f] on v_mfma_f32_16x16x32_bf16, GeGLU in the
//            epilogue, H_e stored as bf16 [rows_e x f];
//   down:    [rows_e x f] x [f x d], fp32 output per (row, slot) pair.
// Each 64x64 weight tile is dequantised once per workgroup (w = s*q + b, fp32,
// rounded to bf16) into LDS and reused by every row tile of the workgroup.
#pragma once

#include "common.h"

namespace qmoe {

// ---------------------------------------------------------------- grouping

// One wavefront. Thread t owns pairs [t*chunk, (t+1)*chunk) in order; cnt[e][t]
// counts them per expert, is turned into per-(expert, thread) start positions
// by an exclusive scan in (expert, thread) order, and every thread then places
// its own pairs in order: a stable counting sort, bit-exact.
__global__ __launch_bounds__(64) void k_group(const int32_t* __restrict__ topk_idx, int n_pairs, int n_experts,
                                              int32_t* __restrict__ count, int32_t* __restrict__ offset,
                                              int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm) {
  extern __shared__ uint16_t cnt[];  // [n_experts][64]
  const int t = threadIdx.x;
  const int chunk = (n_pairs + 63) / 64;
  for (int i = t; i < n_experts * 64; i += 64) cnt[i] = 0;
  __syncthreads();
  const int p0 = t * chunk, p1 = min(n_pairs, p0 + chunk);
  for (int p = p0; p < p1; ++p) {
    const int e = topk_idx[p];
    if (e < 0 || e >= n_experts) {  // not an expert id: reported, and the pair is dropped
      flag_device_error(2u);
      continue;
    }
    cnt[e * 64 + t] += 1;
  }
  __syncthreads();
  __shared__ int32_t tot[257];
  for (int e = t; e < n_experts; e += 64) {
    int s = 0;
    for (int j = 0; j < 64; ++j) s += cnt[e * 64 + j];
    tot[e] = s;
  }
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int e = 0; e < n_experts; ++e) {
      const int c = tot[e];
      count[e] = c;
      offset[e] = run;
      tot[e] = run;
      run += c;
    }
    offset[n_experts] = run;
  }
  __syncthreads();
  for (int e = t; e < n_experts; e += 64) {
    int run = tot[e];
    for (int j = 0; j < 64; ++j) {
      const int c = cnt[e * 64 + j];
      cnt[e * 64 + j] = (uint16_t)run;  // starts fit: n_pairs < 65536 is checked on the host
      run += c;
    }
  }
  __syncthreads();
  for (int p = p0; p < p1; ++p) {
    const int e = topk_idx[p];
    if (e < 0 || e >= n_experts) {
      inv_perm[p] = -1;
      continue;
    }
    const int pos = cnt[e * 64 + t];
    cnt[e * 64 + t] = (uint16_t)(pos + 1);
    perm[pos] = p;
    inv_perm[p] = pos;
  }
}

// ---------------------------------------------------------------- GEMM helpers

constexpr int kLdsStride = 72;  // bf16 per LDS row: 64 + 8 padding (144 B) against bank conflicts

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
  uint16_t* H;            // routed GeGLU output, bf16 [rows*top_k][f] (sorted-pair order)
  uint16_t* Hs;           // shared GeGLU output, bf16 [rows][fs]
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
      T.blob = expert_blob(A.pool, A.stride, A.n_blobs, A.slot_table, e);
      return T.blob != nullptr;
    }
    t += nt;
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const __bf16 ha = (__bf16)a, hb = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// Dequantise 16 consecutive columns (two code words) of one row to bf16 and store
// them to LDS row `dst` at column `col0` (w = s*q + b in fp32, RNE to bf16).
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
      out[t] = pack_bf16x2(fmaf(s, q0, b), fmaf(s, q1, b));
    }
    *reinterpret_cast<uint4*>(dst_row + col0 + 8 * i) = make_uint4(out[0], out[1], out[2], out[3]);
  }
}

__device__ __forceinline__ bf16x8_t lds_frag(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}

// stage 16 columns of activation row `src` (bf16 or fp32) as bf16 hi (+ lo) into LDS
__device__ __forceinline__ void stage_x16(const uint16_t* src, uint16_t* hi, uint16_t*) {
  const uint4* s = reinterpret_cast<const uint4*>(src);
  reinterpret_cast<uint4*>(hi)[0] = s[0];
  reinterpret_cast<uint4*>(hi)[1] = s[1];
}
__device__ __forceinline__ void stage_x16(const float* src, uint16_t* hi, uint16_t* lo) {
  uint32_t h[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = src[2 * i], b = src[2 * i + 1];
    const __bf16 ha = (__bf16)a, hb = (__bf16)b;
    h[i] = (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
    l[i] = pack_bf16x2(a - (float)ha, b - (float)hb);
  }
  reinterpret_cast<uint4*>(hi)[0] = make_uint4(h[0], h[1], h[2], h[3]);
  reinterpret_cast<uint4*>(hi)[1] = make_uint4(h[4], h[5], h[6], h[7]);
  reinterpret_cast<uint4*>(lo)[0] = make_uint4(l[0], l[1], l[2], l[3]);
  reinterpret_cast<uint4*>(lo)[1] = make_uint4(l[4], l[5], l[6], l[7]);
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
  }
  __syncthreads();

  // weight pieces this thread dequantises: matrix wmat, row wr of the 32, 16 columns
  const int wmat = tid >> 7;
  const int wr = (tid & 127) >> 2;
  const int piece = tid & 3;  // half = piece >> 1, words (piece & 1) * 2 .. +1
  const int f0 = fc * 32;
  const int trow = (f0 & 63) + wr;  // row inside the 64-row tile
  const uint8_t* wbase = T.blob + (uint64_t)wmat * m4_bytes(T.F, A.d) + (uint64_t)(f0 >> 6) * G * kTile4;
  // activation pieces: row xr, 16 columns
  const int xr = tid >> 2, xq = tid & 3;
  const int xsrc = rowsrc[xr];

  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int g = 0; g < G; ++g) {
    {  // weights -> LDS (bf16)
      const uint8_t* tile = wbase + (uint64_t)g * kTile4;
      const int h = piece >> 1, jj = (piece & 1) * 2;
      const uint2 cw = *reinterpret_cast<const uint2*>(tile + h * 1024 + trow * 16 + jj * 4);
      const uint32_t sbw = ldg4(tile + kTile4Codes + trow * 4);
      dequant16_to_lds(cw, sbw, &W[wmat][wr * kLdsStride], h * 32 + jj * 8);
    }
    {  // activations -> LDS
      uint16_t* hi = &Xh[xr * kLdsStride + xq * 16];
      uint16_t* lo = kLo ? &Xl[xr * kLdsStride + xq * 16] : nullptr;
      if (xsrc >= 0) {
        stage_x16(x + (size_t)xsrc * A.d + g * kGroup + xq * 16, hi, lo);
      } else {
        reinterpret_cast<uint4*>(hi)[0] = make_uint4(0, 0, 0, 0);
        reinterpret_cast<uint4*>(hi)[1] = make_uint4(0, 0, 0, 0);
        if (kLo) {
          reinterpret_cast<uint4*>(lo)[0] = make_uint4(0, 0, 0, 0);
          reinterpret_cast<uint4*>(lo)[1] = make_uint4(0, 0, 0, 0);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int kc = kk * 32 + 8 * (lane >> 4);
      bf16x8_t bfr[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) bfr[m] = lds_frag(&W[m][(16 * wn + (lane & 15)) * kLdsStride + kc]);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int row = 32 * wm + 16 * mb + (lane & 15);
        const bf16x8_t afr = lds_frag(&Xh[row * kLdsStride + kc]);
#pragma unroll
        for (int m = 0; m < 2; ++m) acc[mb][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[m], acc[mb][m], 0, 0, 0);
        if (kLo) {
          const bf16x8_t alo = lds_frag(&Xl[row * kLdsStride + kc]);
#pragma unroll
          for (int m = 0; m < 2; ++m)
            acc[mb][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bfr[m], acc[mb][m], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }
  // GeGLU epilogue: lane holds rows 4*(lane/16) + i of each 16-row block, column lane % 16
  uint16_t* H = (T.e >= 0) ? A.H : A.Hs;
  const int F = T.F;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 32 * wm + 16 * mb + 4 * (lane >> 4) + i;
      if (r < T.mrows) {
        const float h = gelu_tanh(acc[mb][0][i]) * acc[mb][1][i];
        const __bf16 hb = (__bf16)h;
        H[(size_t)(T.m0 + r) * F + f0 + 16 * wn + (lane & 15)] = __builtin_bit_cast(uint16_t, hb);
      }
    }
}

// ---------------------------------------------------------------- down

// Workgroup = (64-row tile, 64 output columns). 4 waves: wave (wm, wn) owns rows
// [32 wm, +32) and columns [32 wn, +32). grid.x = mtiles * d/64.
__global__ __launch_bounds__(256) void k_prefill_down(PrefillArgs A, int shared) {
  __shared__ __attribute__((aligned(16))) uint16_t Hl[64 * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t W[64 * kLdsStride];
  const int NBd = A.d / 64;
  const int mt = blockIdx.x / NBd;
  const int nb = blockIdx.x % NBd;
  MTile T;
  if (!find_mtile(A, shared != 0, mt, T)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int F = T.F, G = F / kGroup;
  const uint16_t* Hsrc = (T.e >= 0) ? A.H : A.Hs;
  const uint8_t* wbase = T.blob + 2 * m4_bytes(F, A.d) + (uint64_t)nb * G * kTile4;
  const int wr = tid >> 2, piece = tid & 3;
  const int hr = tid >> 2, hq = tid & 3;

  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int g = 0; g < G; ++g) {
    {
      const uint8_t* tile = wbase + (uint64_t)g * kTile4;
      const int h = piece >> 1, jj = (piece & 1) * 2;
      const uint2 cw = *reinterpret_cast<const uint2*>(tile + h * 1024 + wr * 16 + jj * 4);
      const uint32_t sbw = ldg4(tile + kTile4Codes + wr * 4);
      dequant16_to_lds(cw, sbw, &W[wr * kLdsStride], h * 32 + jj * 8);
    }
    {
      uint4* dst = reinterpret_cast<uint4*>(&Hl[hr * kLdsStride + hq * 16]);
      if (hr < T.mrows) {
        const uint4* s = reinterpret_cast<const uint4*>(Hsrc + (size_t)(T.m0 + hr) * F + g * kGroup + hq * 16);
        dst[0] = s[0];
        dst[1] = s[1];
      } else {
        dst[0] = make_uint4(0, 0, 0, 0);
        dst[1] = make_uint4(0, 0, 0, 0);
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int kc = kk * 32 + 8 * (lane >> 4);
      bf16x8_t bfr[2];
#pragma unroll
      for (int nbk = 0; nbk < 2; ++nbk) bfr[nbk] = lds_frag(&W[(32 * wn + 16 * nbk + (lane & 15)) * kLdsStride + kc]);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8_t afr = lds_frag(&Hl[(32 * wm + 16 * mb + (lane & 15)) * kLdsStride + kc]);
#pragma unroll
        for (int nbk = 0; nbk < 2; ++nbk)
          acc[mb][nbk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[nbk], acc[mb][nbk], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  float* out = (T.e >= 0) ? A.expert_out : A.shared_out;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nbk = 0; nbk < 2; ++nbk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 32 * wm + 16 * mb + 4 * (lane >> 4) + i;
        if (r < T.mrows) out[(size_t)(T.m0 + r) * A.d + nb * 64 + 32 * wn + 16 * nbk + (lane & 15)] = acc[mb][nbk][i];
      }
}

// ---------------------------------------------------------------- combine

// y[r][n] = S[r][n] + sum_k w[r][k] * E[pos(r, k)][n], k in slot order; optional residual.
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ shared_out,
                                                 const float* __restrict__ expert_out,
                                                 const int32_t* __restrict__ inv_perm,
                                                 const float* __restrict__ topk_w, int rows, int d, int top_k,
                                                 float* __restrict__ y, uint16_t* __restrict__ residual) {
  const int r = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= d) return;
  float v = shared_out[(size_t)r * d + n];
  for (int k = 0; k < top_k; ++k) {
    const int pos = inv_perm ? inv_perm[r * top_k + k] : r * top_k + k;
    v = fmaf(topk_w[r * top_k + k], expert_out[(size_t)pos * d + n], v);
  }
  y[(size_t)r * d + n] = v;
  if (residual) {
    const float t = bf16_to_f32(residual[(size_t)r * d + n]) + v;
    residual[(size_t)r * d + n] = (uint16_t)f32_to_bf16_bits(t);
  }
}

}  // namespace qmoe
