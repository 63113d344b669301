// Prefill grouped GEMMs on MFMA: each expert's rows (contiguous after grouping)
// against that expert's weights, one fetch of a weight tile serving every row of
// the workgroup's row tile.
//   gate/up: [rows_e x d] x [d x 2*f] on v_mfma_f32_16x16x32_bf16, GeGLU in the
//            epilogue, H_e kept in fp32 [rows_e x f];
//   H pass:  each H row scaled by a power of two and rounded to fp16;
//   down:    [rows_e x f] x [f x d] on v_mfma_f32_16x16x32_f16, fp32 output per
//            (row, slot) pair.
//
// The 4-bit weights are not dequantised element by element. The affine form is
// factored out of the contraction per group of 64 columns:
//   sum_i (s q_i + b) a_i = s * sum_i c_i a_i + (b - s c0) * A_g,   c_i = c0 + q_i,
// where A_g is the group sum of the activations. MFMA computes sum_i c_i a_i and
// A_g (a product with a column of ones) per group from the very operands it
// multiplies; the epilogue applies s and b. Codes and activations enter exactly:
//   gate/up: x is bf16 (exact; fp32 x is split into two bf16 terms hi + lo),
//            c_i = 128 + q_i as bf16 from one mask-and-or per code pair (c0 = 128);
//   down:    H rows scaled so their largest |h| lands in [2^14, 2^15) and rounded
//            to fp16 (11 bits), c_i = q_i as exact fp16 (c0 = 0), and the
//            scale divided out at the end (exactly: a power of two).
//
// Each wavefront loads its own weight fragments straight from the packed tiles
// (the tile layout gives lane l the code word of row l%16, columns 8*(l/16)..+7)
// with kRing groups in flight. Activation tiles are fetched several groups ahead
// into registers, staged once per group in double-buffered LDS and shared by the
// workgroup's four waves.
#pragma once

#include <type_traits>

#include "common.h"

namespace qmoe {

constexpr int kLdsStride = 72;  // halfs per LDS row: 64 + 8 padding (144 B) against bank conflicts
constexpr int kRing = 4;        // weight groups in flight per wavefront
constexpr int kXcds = 8;        // accelerator dies, each with its own L2

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
// native 128-bit vector (HIP's uint4 is a struct: copies of it through register
// arrays become private-memory copies that stay in scratch)

// f(integral_constant<int, i>) for i = 0..N-1: ring slots must be compile-time
// indices, or the register arrays that hold them are demoted to scratch memory
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

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
  float* H;               // routed GeGLU output, fp32 [rows*top_k][f] (sorted-pair order)
  float* Hs;              // shared GeGLU output, fp32 [rows][fs]
  float* hmaxp;           // max |h| per (row, 64-column block): routed [rows*top_k][f/64], then shared [rows][fs/64]
  uint16_t* Hh;           // fp16 of h * hsc: routed [rows*top_k][f], then shared [rows][fs]
  float* hsc;             // power-of-two row scale of Hh: routed [rows*top_k], then shared [rows]
  float* expert_out;      // [rows*top_k][d]
  float* shared_out;      // [rows][d]
};

// 64-row tile -> (expert, first sorted position, row count); expert -1 = shared
struct MTile {
  int e, m0, mrows;
  const uint8_t* blob;
  int F;
};

// Routed tiles are numbered expert by expert (ceil(count_e / 64) tiles each). Each
// lane of a wavefront keeps the ranges of experts [l*epl, (l+1)*epl) (epl <= 4)
// and the prefix of their tile counts, so a tile is found with one ballot.
struct TileMap {
  int excl, incl;  // tiles of the experts before this lane's, and including them
  int off[4], cnt[4];
};

// Fills the map from the grouping offsets; returns the number of routed tiles.
__device__ __forceinline__ int tile_map_init(const PrefillArgs& A, TileMap& M) {
  const int lane = threadIdx.x & 63;
  const int epl = A.n_experts / 64;
  int mine = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    M.off[j] = M.cnt[j] = 0;
    if (j < epl) {
      const int e = lane * epl + j;
      M.off[j] = A.offset[e];
      M.cnt[j] = A.offset[e + 1] - M.off[j];
      mine += (M.cnt[j] + 63) >> 6;
    }
  }
  int incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  M.excl = incl - mine;
  M.incl = incl;
  return __builtin_amdgcn_readfirstlane(__shfl(incl, 63, 64));
}

// 64-row tile -> (expert, first sorted position, row count, weights); every lane
// returns the same tile. False for an expert with no resident weights.
__device__ __forceinline__ bool tile_at(const PrefillArgs& A, const TileMap& M, int mt, MTile& T) {
  const int lane = threadIdx.x & 63;
  const uint64_t hit = __ballot(mt >= M.excl && mt < M.incl);
  if (hit == 0) return false;
  const int owner = __ffsll((unsigned long long)hit) - 1;
  int e = 0, m0 = 0, mr = 0;
  if (lane == owner) {
    const int epl = A.n_experts / 64;
    int t = M.excl;
    bool found = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int nt = (M.cnt[j] + 63) >> 6;
      if (j < epl && !found && mt < t + nt) {
        found = true;
        e = lane * epl + j;
        m0 = M.off[j] + 64 * (mt - t);
        mr = min(64, M.cnt[j] - 64 * (mt - t));
      }
      t += nt;
    }
  }
  // uniform values: kept in scalar registers, so the weight addresses are scalar bases
  T.e = __builtin_amdgcn_readfirstlane(__shfl(e, owner, 64));
  T.m0 = __builtin_amdgcn_readfirstlane(__shfl(m0, owner, 64));
  T.mrows = __builtin_amdgcn_readfirstlane(__shfl(mr, owner, 64));
  T.F = A.f;
  T.blob = uniform_ptr(expert_blob(A.pool, A.stride, A.n_blobs, A.slot_table, T.e, A.n_experts, true));
  return T.blob != nullptr;
}

__device__ __forceinline__ void shared_tile(const PrefillArgs& A, int mt, MTile& T) {
  T.e = -1;
  T.m0 = 64 * mt;
  T.mrows = min(64, A.rows - T.m0);
  T.blob = A.shared_blob;
  T.F = A.fs;
}

// Workgroups are dealt to the XCDs round robin by block index. A section of `nt`
// row tiles x `nc` column blocks is laid out so that all column blocks of one row
// tile land on the same XCD (its activation tile is fetched into that L2 once)
// and consecutive row tiles go to different XCDs. `lanes` = min(kXcds, nt).
__host__ __device__ inline int xcd_lanes(int nt) { return nt < kXcds ? (nt > 0 ? nt : 1) : kXcds; }
__host__ __device__ inline int xcd_blocks(int nt, int nc) {
  const int k = xcd_lanes(nt);
  return (nt + k - 1) / k * k * nc;
}
__device__ __forceinline__ void xcd_item(int b, int nt, int nc, int& mt, int& c) {
  const int k = xcd_lanes(nt);
  const int per = k * nc;
  const int q = b / per, r = b - q * per;
  mt = q * k + r % k;
  c = r / k;
}


// B operand, gate/up: the 8 codes of one packed word as bf16 (128 + q)
__device__ __forceinline__ bf16x8_t codes_bf16(uint32_t w, const NibK& nk) {
  const u32x4_t p = {nk.pair(w, 0), nk.pair(w, 1), nk.pair(w, 2), nk.pair(w, 3)};
  return __builtin_bit_cast(bf16x8_t, p);
}

// B operand, down: the 8 codes of one packed word as exact fp16 values q (0..15):
// the pair (1024 + q, 1024 + q') is built with a mask and an OR of the exponent of
// 1024 (0x6400), then 1024 is subtracted with one packed fp16 add per pair.
__device__ __forceinline__ f16x8_t codes_f16(uint32_t w, const NibKT<0x64006400u>& mk) {
  const f16x2_t k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  f16x2_t p[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) p[t] = __builtin_bit_cast(f16x2_t, ((w >> (4 * t)) & mk.mask) | mk.expo) - k1024;
  return f16x8_t{p[0].x, p[0].y, p[1].x, p[1].y, p[2].x, p[2].y, p[3].x, p[3].y};
}

template <typename V>
__device__ __forceinline__ V lds_frag(const uint16_t* p) {
  return __builtin_bit_cast(V, *reinterpret_cast<const u32x4_t*>(p));
}

__device__ __forceinline__ f32x4_t mfma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma(f16x8_t a, f16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Weight fragments of NM matrices in a ring of kRing groups: for wave row `row`
// (0..63 within the 64-row block), the two code words of k-halves 0 and 1 and the
// (scale, bias) pair, from tile g of the column block whose tiles start at the base
// of wres[m]. The lane offsets are fixed; the group enters as a scalar offset.
template <int NM>
struct BRing {
  uint32_t cw[kRing][NM][2];
  uint32_t sb[kRing][NM];
  uint32_t vc, vs;  // lane offsets of the code word and of (s, b) within a tile
  __device__ __forceinline__ void init(int row, int lane) {
    vc = row * 16 + (lane >> 4) * 4;
    vs = kTile4Codes + row * 4;
  }
  template <int slot>
  __device__ __forceinline__ void load(ic<slot>, const rsrc_t* wres, int g) {
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const uint32_t so = (uint32_t)g * kTile4;
      cw[slot][m][0] = bld4(wres[m], vc, so);
      cw[slot][m][1] = bld4(wres[m], vc + 1024, so);
      sb[slot][m] = bld4(wres[m], vs, so);
    }
  }
};

__device__ __forceinline__ void zero_acc(f32x4_t& a) { a = f32x4_t{0.f, 0.f, 0.f, 0.f}; }


// ---------------------------------------------------------------- gate/up + GeGLU

// LDS of the gate/up kernel: double-buffered activation tiles (bf16 hi, and lo for
// fp32 x) and the per-wave row maxima of |h|
template <bool LO>
struct GateupSmem {
  __attribute__((aligned(16))) uint16_t Xs[2][64 * kLdsStride];
  __attribute__((aligned(16))) uint16_t Xls[LO ? 2 : 1][LO ? 64 * kLdsStride : 8];
  float hmL[4][64];
};

// One work item = (64-row tile, 64 d_ff columns). Wave w owns d_ff columns [16w, +16)
// of both gate and up (so GeGLU runs in registers) for every row of the tile.
template <typename XT>
__device__ __forceinline__ void gateup_tile(const PrefillArgs& A, const XT* __restrict__ x, const MTile& T, int fc,
                                            bool shared, GateupSmem<sizeof(XT) == 4>& S) {
  constexpr bool LO = sizeof(XT) == 4;  // fp32 x: hi + lo bf16 terms
  constexpr int RA = LO ? 2 : 4;        // activation groups in flight
  constexpr int NV = LO ? 4 : 2;        // 16-byte loads per thread per group
  auto& Xs = S.Xs;
  auto& Xls = S.Xls;
  auto& hmL = S.hmL;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = A.d / kGroup;
  const int nmb = (T.mrows + 15) >> 4;

  // weight rows of this wave: row 16*wave + lane%16 of the 64-row block fc of gate and up
  const int wrow = 16 * wave + (lane & 15);
  rsrc_t wres[2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
    wres[m] = buf_rsrc(uniform_ptr(T.blob) + (uint64_t)m * m4_bytes(T.F, A.d) + (uint64_t)fc * G * kTile4,
                       (uint32_t)G * kTile4);
  BRing<2> B;
  B.init(wrow, lane);

  // activation staging: thread -> tile row tid/4, 16 values at column (tid%4)*16.
  // Rows past the tile's end repeat its first row: MFMA output rows depend on their
  // own A rows only, and those rows are never stored, so the loads need no branch.
  const int xr = tid >> 2, xq = tid & 3;
  const int xt = xr < T.mrows ? xr : 0;
  const int xsrc = T.e >= 0 ? A.perm[T.m0 + xt] / A.top_k : T.m0 + xt;
  const rsrc_t xres = buf_rsrc(x, (uint32_t)((size_t)A.rows * A.d * sizeof(XT)));
  const uint32_t xvo = (uint32_t)(((size_t)xsrc * A.d + xq * 16) * sizeof(XT));
  u32x4_t xa[RA][NV];
  auto aload = [&](auto sc, int g) __attribute__((always_inline)) {
    constexpr int slot = decltype(sc)::value;
#pragma unroll
    for (int v = 0; v < NV; ++v) xa[slot][v] = bld16(xres, xvo + 16 * v, (uint32_t)(g * kGroup * sizeof(XT)));
  };
  auto astore = [&](auto sc, int buf) __attribute__((always_inline)) {
    constexpr int slot = decltype(sc)::value;
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(&Xs[buf][xr * kLdsStride + xq * 16]);
    if (!LO) {
      dst[0] = xa[slot][0];
      dst[1] = xa[slot][1];
    } else {
      // 16 fp32 values -> bf16 hi (round to nearest even) and bf16 lo of the remainder
      uint32_t hi[8], lo[8];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint32_t w[4] = {xa[slot][v].x, xa[slot][v].y, xa[slot][v].z, xa[slot][v].w};
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          uint32_t h2 = 0, l2 = 0;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const float f = __uint_as_float(w[2 * p + q]);
            const uint32_t hb = f32_to_bf16_bits(f);
            const uint32_t lb = f32_to_bf16_bits(f - __uint_as_float(hb << 16));
            h2 |= hb << (16 * q);
            l2 |= lb << (16 * q);
          }
          hi[2 * v + p] = h2;
          lo[2 * v + p] = l2;
        }
      }
      u32x4_t* dl = reinterpret_cast<u32x4_t*>(&Xls[buf][xr * kLdsStride + xq * 16]);
      dst[0] = u32x4_t{hi[0], hi[1], hi[2], hi[3]};
      dst[1] = u32x4_t{hi[4], hi[5], hi[6], hi[7]};
      dl[0] = u32x4_t{lo[0], lo[1], lo[2], lo[3]};
      dl[1] = u32x4_t{lo[4], lo[5], lo[6], lo[7]};
    }
  };
  // prologue: the loads in the order the steady state issues them (weights of group
  // j, then activations of group j + 1), so the wait counts agree on entry
  aload(ic<0>{}, 0);
  static_for<kRing>([&](auto jc) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    B.load(jc, wres, min(j, G - 1));
    if constexpr (j + 1 < RA) aload(ic<j + 1>{}, min(j + 1, G - 1));
    if constexpr (j + 1 == RA) {
      astore(ic<0>{}, 0);
      aload(ic<0>{}, min(RA, G - 1));
    }
  });
  __syncthreads();

  // The compute is compiled for NMB = 1, 2 and 4 blocks of 16 rows (3 runs as 4), so
  // the blocks' MFMAs and epilogue FMAs form straight-line code the scheduler can
  // interleave, instead of one branch per block.
  auto run = [&](auto nc) __attribute__((always_inline)) {
    constexpr int NMB = decltype(nc)::value;
    f32x4_t acc[NMB][2];
  #pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      zero_acc(acc[mb][0]);
      zero_acc(acc[mb][1]);
    }
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});

    // One K group: MFMAs from LDS buffer j&1 and weight slot j; then the weight
    // slot is refilled with group g + kRing and the activation slot staged next is
    // refilled with group g + 1 + RA, both clamped to the last group (the surplus
    // loads near the end are never used). The steady-state loop is
    // straight-line code over kRing groups, so every ring slot keeps its own
    // registers and no wait covers a load younger than the one it needs.
    const NibK nk;
    auto step = [&](auto jc, int g) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      constexpr int buf = j & 1;
      bf16x8_t bfr[2][2];
      float s[2], bb[2];
  #pragma unroll
      for (int m = 0; m < 2; ++m) {
        bfr[m][0] = codes_bf16(B.cw[j][m][0], nk);
        bfr[m][1] = codes_bf16(B.cw[j][m][1], nk);
        s[m] = bf16_lo(B.sb[j][m]);
        bb[m] = fmaf(-128.0f, s[m], bf16_hi(B.sb[j][m]));  // b - 128 s
      }
      B.load(jc, wres, min(g + kRing, G - 1));
  #pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        {
          const int ao = (16 * mb + (lane & 15)) * kLdsStride + 8 * (lane >> 4);
          const bf16x8_t a0 = lds_frag<bf16x8_t>(&Xs[buf][ao]);
          const bf16x8_t a1 = lds_frag<bf16x8_t>(&Xs[buf][ao + 32]);
          f32x4_t ag = mfma(a1, ones, mfma(a0, ones, f32x4_t{0.f, 0.f, 0.f, 0.f}));
          f32x4_t t[2];
  #pragma unroll
          for (int m = 0; m < 2; ++m) t[m] = mfma(a1, bfr[m][1], mfma(a0, bfr[m][0], f32x4_t{0.f, 0.f, 0.f, 0.f}));
          if (LO) {
            const bf16x8_t l0 = lds_frag<bf16x8_t>(&Xls[buf][ao]);
            const bf16x8_t l1 = lds_frag<bf16x8_t>(&Xls[buf][ao + 32]);
            ag = mfma(l1, ones, mfma(l0, ones, ag));
  #pragma unroll
            for (int m = 0; m < 2; ++m) t[m] = mfma(l1, bfr[m][1], mfma(l0, bfr[m][0], t[m]));
          }
  #pragma unroll
          for (int m = 0; m < 2; ++m)
  #pragma unroll
            for (int i = 0; i < 4; ++i) acc[mb][m][i] = fmaf(s[m], t[m][i], fmaf(bb[m], ag[i], acc[mb][m][i]));
        }
      }
      // next activation group into the other buffer (its readers passed the last barrier)
      astore(ic<(j + 1) % RA>{}, buf ^ 1);
      aload(ic<(j + 1) % RA>{}, min(g + 1 + RA, G - 1));
      __syncthreads();
    };
    int g0 = 0;
    for (; g0 + kRing <= G; g0 += kRing) {
      step(ic<0>{}, g0);
      step(ic<1>{}, g0 + 1);
      step(ic<2>{}, g0 + 2);
      step(ic<3>{}, g0 + 3);
    }
    // the last G % kRing groups
    if (g0 < G) step(ic<0>{}, g0);
    if (g0 + 1 < G) step(ic<1>{}, g0 + 1);
    if (g0 + 2 < G) step(ic<2>{}, g0 + 2);

    // GeGLU epilogue: lane holds rows 16mb + 4*(lane/16) + i, d_ff column fc*64 + 16*wave + lane%16
    float* H = shared ? A.Hs : A.H;
    float* hmaxp = shared ? A.hmaxp + (size_t)A.rows * A.top_k * (A.f / 64) : A.hmaxp;
    const int F = T.F, nG = F / 64;
  #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mb + 4 * (lane >> 4) + i;
        float h = 0.0f;
        if (r < T.mrows) {
          h = gelu_tanh(acc[mb][0][i]) * acc[mb][1][i];
          H[(size_t)(T.m0 + r) * F + fc * 64 + 16 * wave + (lane & 15)] = h;
        }
        // max |h| over the 16 lanes holding this row: one DPP row (VALU, no LDS round trips)
        const float mx = row16_max(fabsf(h));
        if ((lane & 15) == 0) hmL[wave][r] = mx;
      }
    __syncthreads();
    if (tid < T.mrows)
      hmaxp[(size_t)(T.m0 + tid) * nG + fc] = fmaxf(fmaxf(hmL[0][tid], hmL[1][tid]), fmaxf(hmL[2][tid], hmL[3][tid]));

  };
  if (nmb == 1)
    run(ic<1>{});
  else if (nmb == 2)
    run(ic<2>{});
  else
    run(ic<4>{});
}

// Persistent: a grid sized to what the chip holds at once walks the work items
// (shared-expert items first: they are the longest; then the routed tiles that
// exist), so no workgroup slot goes to an empty tile.
template <typename XT>
__global__ __launch_bounds__(256, 2) void k_prefill_gateup(PrefillArgs A, const XT* __restrict__ x) {
  __shared__ GateupSmem<sizeof(XT) == 4> S;
  TileMap M;
  const int nrt = A.routed_mtiles > 0 ? tile_map_init(A, M) : 0;
  const int ncs = A.fs / 64, ncr = A.f / 64;
  const int ns = xcd_blocks(A.shared_mtiles, ncs);
  const int n = ns + xcd_blocks(nrt, ncr);
  for (int item = blockIdx.x; item < n; item += gridDim.x) {
    const bool shared = item < ns;
    int mt, fc;
    MTile T;
    if (shared) {
      xcd_item(item, A.shared_mtiles, ncs, mt, fc);
      if (mt >= A.shared_mtiles) continue;
      shared_tile(A, mt, T);
    } else {
      xcd_item(item - ns, nrt, ncr, mt, fc);
      if (mt >= nrt || !tile_at(A, M, mt, T)) continue;
    }
    gateup_tile<XT>(A, x, T, fc, shared, S);
    __syncthreads();  // the next item reuses the LDS
  }
}

// ---------------------------------------------------------------- H to fp16

// One wavefront per H row (rows [first, first + count) of the routed rows followed
// by the shared rows): the row's power-of-two scale from its per-block maxima, then
// the fp16 copy of h * scale. Every load of a round (the maxima and up to
// kHconvLoads 16-byte pieces of the row per lane) is issued before any is used.
constexpr int kHconvLoads = 9;
__global__ __launch_bounds__(256) void k_prefill_hconv(PrefillArgs A, int first, int count) {
  const int lane = threadIdx.x & 63;
  const int r = first + (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (r >= first + count) return;
  const int P = A.rows * A.top_k;
  const float* src;
  const float* mp;
  uint16_t* dst;
  int F;
  if (r < P) {
    F = A.f;
    src = A.H + (size_t)r * F;
    mp = A.hmaxp + (size_t)r * (F / 64);
    dst = A.Hh + (size_t)r * F;
  } else {
    const int rs = r - P;
    F = A.fs;
    src = A.Hs + (size_t)rs * F;
    mp = A.hmaxp + (size_t)P * (A.f / 64) + (size_t)rs * (F / 64);
    dst = A.Hh + (size_t)P * A.f + (size_t)rs * F;
  }
  const int nG = F / 64;
  const rsrc_t hres = buf_rsrc(src, (uint32_t)F * 4u);  // loads past the row return 0
  float m = 0.0f;
  for (int c0 = 0; c0 < F; c0 += 256 * kHconvLoads) {
    u32x4_t v[kHconvLoads];
#pragma unroll
    for (int j = 0; j < kHconvLoads; ++j) v[j] = bld16(hres, (uint32_t)(c0 + 256 * j + 4 * lane) * 4u, 0);
    if (c0 == 0) {
      for (int i = lane; i < nG; i += 64) m = fmaxf(m, mp[i]);
      m = wave_fmax(m);
    }
    const float sc = row_scale(m);
    if (c0 == 0 && lane == 0) A.hsc[r] = sc;
#pragma unroll
    for (int j = 0; j < kHconvLoads; ++j) {
      const int c = c0 + 256 * j + 4 * lane;
      if (c < F) {
        const uint32_t p0 = (uint32_t)f16_bits(__uint_as_float(v[j][0]) * sc) |
                            ((uint32_t)f16_bits(__uint_as_float(v[j][1]) * sc) << 16);
        const uint32_t p1 = (uint32_t)f16_bits(__uint_as_float(v[j][2]) * sc) |
                            ((uint32_t)f16_bits(__uint_as_float(v[j][3]) * sc) << 16);
        *reinterpret_cast<uint2*>(dst + c) = make_uint2(p0, p1);
      }
    }
  }
}

// ---------------------------------------------------------------- down

struct DownSmem {
  __attribute__((aligned(16))) uint16_t Hl[2][64 * kLdsStride];
  float rowinv[64];
  __attribute__((aligned(16))) float agL[2][64];  // per-row sums of the staged H group
};

// One work item = (64-row tile, two blocks of 64 output columns, 2 np and 2 np + 1).
// Wave w owns output columns [16w, +16) of both blocks for every row of the tile, so
// one staged H tile feeds twice the columns. With an odd number of blocks the last
// item's second block repeats its first and is not stored.
constexpr int kDownBlocks = 2;
__device__ __forceinline__ void down_tile(const PrefillArgs& A, const MTile& T, int np, bool shared, DownSmem& S) {
  constexpr int RA = 4;
  auto& Hl = S.Hl;
  auto& rowinv = S.rowinv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int F = T.F, G = F / kGroup;
  const int nmb = (T.mrows + 15) >> 4;
  const int P = A.rows * A.top_k;
  const uint16_t* Hh = shared ? A.Hh + (size_t)P * A.f : A.Hh;
  const float* hsc = shared ? A.hsc + P : A.hsc;

  const int wrow = 16 * wave + (lane & 15);
  const int nblk = A.d / 64;
  int nbm[kDownBlocks];
  rsrc_t wres[kDownBlocks];
#pragma unroll
  for (int m = 0; m < kDownBlocks; ++m) {
    nbm[m] = min(kDownBlocks * np + m, nblk - 1);
    wres[m] = buf_rsrc(uniform_ptr(T.blob) + 2 * m4_bytes(F, A.d) + (uint64_t)nbm[m] * G * kTile4,
                       (uint32_t)G * kTile4);
  }
  BRing<kDownBlocks> B;
  B.init(wrow, lane);
  if (tid < 64) rowinv[tid] = tid < T.mrows ? 1.0f / hsc[T.m0 + tid] : 1.0f;  // exact: powers of two

  // H staging: thread -> tile row tid/4, 16 halfs at column (tid%4)*16; rows past
  // the tile's end repeat its first row (see the gate/up kernel)
  const int hr = tid >> 2, hq = tid & 3;
  const rsrc_t hres = buf_rsrc(Hh, (uint32_t)((size_t)(shared ? A.rows : P) * F * sizeof(uint16_t)));
  const uint32_t hvo = (uint32_t)(((size_t)(T.m0 + (hr < T.mrows ? hr : 0)) * F + hq * 16) * sizeof(uint16_t));
  u32x4_t ha[RA][2];
  auto aload = [&](auto sc, int g) __attribute__((always_inline)) {
    constexpr int slot = decltype(sc)::value;
    const uint32_t so = (uint32_t)(g * kGroup * sizeof(uint16_t));
    ha[slot][0] = bld16(hres, hvo, so);
    ha[slot][1] = bld16(hres, hvo + 16, so);
  };
  // the staging threads also add up each row's group (dot products against fp16 (1, 1)
  // pairs, the four threads of a row summed by DPP) for the bias term of the epilogue
  auto astore = [&](auto sc, int buf) __attribute__((always_inline)) {
    constexpr int slot = decltype(sc)::value;
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(&Hl[buf][hr * kLdsStride + hq * 16]);
    dst[0] = ha[slot][0];
    dst[1] = ha[slot][1];
    float v = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t w = ha[slot][h][c];  // a bit_cast of the vector element itself reads element 0
        v = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w), __builtin_bit_cast(f16x2_t, 0x3C003C00u), v, false);
      }
    v = dpp_add<0xB1, 0xf>(v);  // the four threads of a row are one quad
    v = dpp_add<0x4E, 0xf>(v);
    if (hq == 0) S.agL[buf][hr] = v;
  };
  // prologue: the loads in the order the steady state issues them (weights of group
  // j, then activations of group j + 1), so the wait counts agree on entry
  aload(ic<0>{}, 0);
  static_for<kRing>([&](auto jc) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    B.load(jc, wres, min(j, G - 1));
    if constexpr (j + 1 < RA) aload(ic<j + 1>{}, min(j + 1, G - 1));
    if constexpr (j + 1 == RA) {
      astore(ic<0>{}, 0);
      aload(ic<0>{}, min(RA, G - 1));
    }
  });
  __syncthreads();

  f32x4_t acc[4][kDownBlocks];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int m = 0; m < kDownBlocks; ++m) zero_acc(acc[mb][m]);

  // one K group, as in the gate/up kernel
  const NibKT<0x64006400u> nk;
  auto step = [&](auto jc, int g) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    constexpr int buf = j & 1;
    f16x8_t b0[kDownBlocks], b1[kDownBlocks];
    float s[kDownBlocks], bp[kDownBlocks];
#pragma unroll
    for (int m = 0; m < kDownBlocks; ++m) {
      b0[m] = codes_f16(B.cw[j][m][0], nk);
      b1[m] = codes_f16(B.cw[j][m][1], nk);
      s[m] = bf16_lo(B.sb[j][m]);
      bp[m] = bf16_hi(B.sb[j][m]);
    }
    B.load(jc, wres, min(g + kRing, G - 1));
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      if (mb < nmb) {
        const int ao = (16 * mb + (lane & 15)) * kLdsStride + 8 * (lane >> 4);
        const f16x8_t a0 = lds_frag<f16x8_t>(&Hl[buf][ao]);
        const f16x8_t a1 = lds_frag<f16x8_t>(&Hl[buf][ao + 32]);
        const f32x4_t ag = *reinterpret_cast<const f32x4_t*>(&S.agL[buf][16 * mb + 4 * (lane >> 4)]);
#pragma unroll
        for (int m = 0; m < kDownBlocks; ++m) {
          const f32x4_t t = mfma(a1, b1[m], mfma(a0, b0[m], f32x4_t{0.f, 0.f, 0.f, 0.f}));
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mb][m][i] = fmaf(s[m], t[i], fmaf(bp[m], ag[i], acc[mb][m][i]));
        }
      }
    }
    astore(ic<(j + 1) % RA>{}, buf ^ 1);
    aload(ic<(j + 1) % RA>{}, min(g + 1 + RA, G - 1));
    __syncthreads();
  };
  int g0 = 0;
  for (; g0 + kRing <= G; g0 += kRing) {
    step(ic<0>{}, g0);
    step(ic<1>{}, g0 + 1);
    step(ic<2>{}, g0 + 2);
    step(ic<3>{}, g0 + 3);
  }
  if (g0 < G) step(ic<0>{}, g0);
  if (g0 + 1 < G) step(ic<1>{}, g0 + 1);
  if (g0 + 2 < G) step(ic<2>{}, g0 + 2);
  float* out = shared ? A.shared_out : A.expert_out;
#pragma unroll
  for (int m = 0; m < kDownBlocks; ++m) {
    if (kDownBlocks * np + m >= nblk) break;  // the repeated last block
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mb + 4 * (lane >> 4) + i;
        if (r < T.mrows)
          out[(size_t)(T.m0 + r) * A.d + nbm[m] * 64 + 16 * wave + (lane & 15)] = acc[mb][m][i] * rowinv[r];
      }
  }
}

// Persistent over the work items, as the gate/up kernel.
__global__ __launch_bounds__(256, 2) void k_prefill_down(PrefillArgs A) {
  __shared__ DownSmem S;
  TileMap M;
  const int nrt = A.routed_mtiles > 0 ? tile_map_init(A, M) : 0;
  const int nc = (A.d / 64 + kDownBlocks - 1) / kDownBlocks;
  const int ns = xcd_blocks(A.shared_mtiles, nc);
  const int n = ns + xcd_blocks(nrt, nc);
  for (int item = blockIdx.x; item < n; item += gridDim.x) {
    const bool shared = item < ns;
    int mt, nb;
    MTile T;
    if (shared) {
      xcd_item(item, A.shared_mtiles, nc, mt, nb);
      if (mt >= A.shared_mtiles) continue;
      shared_tile(A, mt, T);
    } else {
      xcd_item(item - ns, nrt, nc, mt, nb);
      if (mt >= nrt || !tile_at(A, M, mt, T)) continue;
    }
    down_tile(A, T, nb, shared, S);
    __syncthreads();  // the next item reuses the LDS
  }
}

}  // namespace qmoe
