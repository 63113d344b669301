// Prefill grouped GEMMs on MFMA: each expert's rows (contiguous after grouping)
// against that expert's weights, one fetch of a weight tile serving every row of
// the workgroup's row tile.
//   gate/up: [rows_e x d] x [d x 2*f] on v_mfma_f32_16x16x32_bf16, GeGLU in the
//            epilogue, H_e stored as fp16 [rows_e x f], each (row, 64-column block)
//            scaled by a power of two kept beside it;
//   down:    [rows_e x f] x [f x d] on v_mfma_f32_16x16x32_f16, fp32 output per
//            (row, slot) pair.
//
// The 4-bit weights are not dequantised element by element. The affine form is
// factored out of the contraction per group of 64 columns:
//   sum_i (s q_i + b) a_i = s * sum_i c_i a_i + (b - s c0) * A_g,   c_i = c0 + q_i,
// where A_g is the group sum of the activations. MFMA computes sum_i c_i a_i per
// group; the epilogue applies s and b. A_g of the gate/up activations is computed
// once per chunk (by the router kernel, or k_group_sums for the split calls) and
// held in LDS per tile; A_g of H comes from the threads that stage each H group.
// Codes and activations enter exactly:
//   gate/up: x is bf16 (exact; fp32 x is split into two bf16 terms hi + lo),
//            c_i = 128 + q_i as bf16 from one mask-and-or per code pair (c0 = 128);
//   down:    H blocks scaled so their largest |h| lands in [2^14, 2^15), rounded to
//            fp16 (11 bits) and brought to one scale per row and item (exact powers
//            of two), c_i = 1024 + q_i as exact fp16 from one mask-and-or per code
//            pair (c0 = 1024), and the scale divided out at the end (exactly).
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
// The shared expert's down projection runs in this many K parts (d_ff_shared / 3 is the
// routed experts' d_ff in the Gemma-like shape), each a work item of its own, so its
// items are no longer than a routed expert's; the combine adds the parts in order.
constexpr int kSharedDownParts = 3;
constexpr int kXcds = 8;        // accelerator dies, each with its own L2
constexpr int kMaxG = 96;       // groups of the reduction: d_model <= 6144


typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
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
  const float* xg;        // group sums of the activations, fp32 [rows][d/64] (the router kernel's)
  uint16_t* Hh;           // GeGLU output h as fp16 of h * hbs: routed [rows*top_k][f] (sorted-pair order),
                          // then shared [rows][fs]
  float* hbs;             // power-of-two scale of each (row, 64-column block) of Hh: routed
                          // [rows*top_k][f/64], then shared [rows][fs/64]
  float* expert_out;      // [rows*top_k][d]
  float* shared_out;      // [kSharedDownParts][rows][d]: the shared expert's down in K parts
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

// B operand, down: the 8 codes of one packed word as exact fp16 values 1024 + q: each
// pair (1024 + q, 1024 + q') is a mask and an OR of the exponent of 1024 (0x6400), and
// 1024 goes into the bias term (b - 1024 s), as in the decode GEMV.
__device__ __forceinline__ f16x8_t codes_f16(uint32_t w, const NibKT<0x64006400u>& mk) {
  f16x2_t p[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) p[t] = __builtin_bit_cast(f16x2_t, ((w >> (4 * t)) & mk.mask) | mk.expo);
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

// Weight fragments of two 64-row blocks (gate and up of one column block, or two output
// blocks of the down projection) in a ring of kDepth groups, for wave row `row` (0..63
// within a block). The matrix cores want, in lane 16c + n, code word c of row n's 16-byte
// segment of each (block, k-half). Those words sit 16 bytes apart, so fetching them
// directly takes four 4-byte loads whose 16-lane quarters each touch 256 bytes. Instead
// every lane fetches one whole 16-byte segment: lanes 16q + n take k-half q & 1 of block
// q >> 1 (16 lanes cover 256 contiguous bytes), and a 4 x 4 transpose across the four
// 16-lane rows (two permlane32 and two permlane16 swaps) gives each lane its words. The
// (scale, bias) words take one load too: 16-lane row q fetches block q & 1's word of its
// row, and one permlane16 swap of that register with itself puts block 0's word in every
// row of one result and block 1's in every row of the other. One buffer resource spans
// both blocks, which start `mstride` bytes apart; the group enters as a scalar offset.
template <int kDepth>
struct BRingT {
  u32x4_t cw[kDepth];  // as fetched; transposed when used
  uint32_t sb[kDepth];
  uint32_t vc, vs;
  __device__ __forceinline__ void init(int row, int lane, uint32_t mstride) {
    vc = (uint32_t)(lane >> 5) * mstride + (uint32_t)((lane >> 4) & 1) * 1024u + (uint32_t)row * 16u;
    vs = (uint32_t)((lane >> 4) & 1) * mstride + kTile4Codes + (uint32_t)row * 4u;
  }
  template <int slot>
  __device__ __forceinline__ void load(ic<slot>, rsrc_t r, int g) {
    const uint32_t so = (uint32_t)g * kTile4;
    cw[slot] = bld16(r, vc, so);
    sb[slot] = bld4(r, vs, so);
  }
  // the (scale, bias) words of a slot: element m is block m's
  template <int slot>
  __device__ __forceinline__ u32x2_t scales(ic<slot>) const {
    const auto t = __builtin_amdgcn_permlane16_swap(sb[slot], sb[slot], false, false);
    return u32x2_t{t[0], t[1]};
  }
  // the code words of a slot: element 2 m + h is k-half h of block m
  template <int slot>
  __device__ __forceinline__ u32x4_t codes(ic<slot>) const {
    u32x4_t w = cw[slot];
    const auto a = __builtin_amdgcn_permlane32_swap(w[0], w[2], false, false);  // rows 2,3 of the first <-> rows 0,1 of the second
    const auto b = __builtin_amdgcn_permlane32_swap(w[1], w[3], false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);  // rows 1,3 of the first <-> rows 0,2 of the second
    const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    return u32x4_t{c[0], c[1], d[0], d[1]};
  }
};
using BRing = BRingT<kRing>;

__device__ __forceinline__ void zero_acc(f32x4_t& a) { a = f32x4_t{0.f, 0.f, 0.f, 0.f}; }


// ---------------------------------------------------------------- gate/up + GeGLU

// LDS of the gate/up kernel: double-buffered activation stages of up to two groups
// (bf16 hi, and lo for fp32 x, whose stages hold one group), the group sums of the
// tile's rows (group-major: xgL[g][row]) and the per-wave row maxima of |h|
template <bool LO>
struct GateupSmem {
  static constexpr int kMaxStage = LO ? 1 : 2;  // groups per stage
  __attribute__((aligned(16))) uint16_t Xs[2 * 64 * (kMaxStage * 64 + 8)];
  __attribute__((aligned(16))) uint16_t Xls[LO ? 2 * 64 * 72 : 8];
  __attribute__((aligned(16))) float xgL[kMaxG * 64];
  float hmL[4][64];
  __attribute__((aligned(16))) float hsL[64];
};

// One work item = (64-row tile, 64 d_ff columns). Wave w owns d_ff columns [16w, +16)
// of both gate and up (so GeGLU runs in registers) for every row of the tile.
// Activations are staged SG groups at a time (one barrier per stage); within a stage
// the K groups need no barrier between them, so the scheduler can overlap one group's
// epilogue with the next group's matrix work. The group sums X_g of the bias term come
// from LDS (filled once per tile from the chunk's precomputed sums), not from MFMAs.
template <typename XT, int SG>
__device__ __forceinline__ void gateup_tile(const PrefillArgs& A, const XT* __restrict__ x, const MTile& T, int fc,
                                            bool shared, GateupSmem<sizeof(XT) == 4>& S) {
  constexpr bool LO = sizeof(XT) == 4;  // fp32 x: hi + lo bf16 terms
  static_assert(!LO || SG == 1, "fp32 activations stage one group at a time");
  static_assert(kRing % SG == 0 && (kRing / SG) % 2 == 0, "stages alternate buffers within the ring");
  constexpr int RA = LO ? 2 : 4;        // activation groups in flight (a multiple of SG)
  constexpr int NV = LO ? 4 : 2;        // 16-byte loads per thread per group
  constexpr int kStride = SG * 64 + 8;  // halfs per staged row: SG groups + 8 padding against bank conflicts
  constexpr int kBuf = 64 * kStride;
  uint16_t* Xs = S.Xs;
  uint16_t* Xls = S.Xls;
  auto& hmL = S.hmL;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = A.d / kGroup;
  const int nmb = (T.mrows + 15) >> 4;

  // weight rows of this wave: row 16*wave + lane%16 of the 64-row block fc of gate and up
  const int wrow = 16 * wave + (lane & 15);
  const uint32_t mstride = (uint32_t)m4_bytes(T.F, A.d);  // gate to up
  const rsrc_t wres = buf_rsrc(uniform_ptr(T.blob) + (uint64_t)fc * G * kTile4, mstride + (uint32_t)G * kTile4);
  BRing B;
  B.init(wrow, lane, mstride);

  // activation staging: thread -> tile row tid/4, 16 values at column (tid%4)*16 of a group.
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
  // ring slot -> its place in a stage buffer (group g sits in slot g % RA, place g % SG)
  auto astore = [&](auto sc, int buf) __attribute__((always_inline)) {
    constexpr int slot = decltype(sc)::value;
    constexpr int pos = slot % SG;
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(&Xs[buf * kBuf + xr * kStride + pos * 64 + xq * 16]);
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
      u32x4_t* dl = reinterpret_cast<u32x4_t*>(&Xls[buf * kBuf + xr * kStride + pos * 64 + xq * 16]);
      dst[0] = u32x4_t{hi[0], hi[1], hi[2], hi[3]};
      dst[1] = u32x4_t{hi[4], hi[5], hi[6], hi[7]};
      dl[0] = u32x4_t{lo[0], lo[1], lo[2], lo[3]};
      dl[1] = u32x4_t{lo[4], lo[5], lo[6], lo[7]};
    }
  };
  // prologue: the loads in the order the steady state issues them (weights of group
  // j, then activations of group j + 1), so the wait counts agree on entry; then the
  // first stage into buffer 0 and its ring slots refilled
  aload(ic<0>{}, 0);
  static_for<kRing>([&](auto jc) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    B.load(jc, wres, min(j, G - 1));
    if constexpr (j + 1 < RA) aload(ic<j + 1>{}, min(j + 1, G - 1));
    if constexpr (j + 1 == RA) {
      static_for<SG>([&](auto pc) __attribute__((always_inline)) {
        constexpr int p = decltype(pc)::value;
        astore(ic<p>{}, 0);
        aload(ic<p>{}, min(RA + p, G - 1));
      });
    }
  });
  // the group sums of the tile's rows into LDS, group-major (rows past the tile's end
  // take row 0's, as the activations do): thread t loads row t%64, groups 4 (t/64 + 4u)
  // .. +3 as one 16-byte load (rows of xg are padded to a multiple of four groups; a
  // load past the array returns zeros), all loads issued before the first store
  {
    const int r = tid & 63;
    const int src = r < T.mrows ? r : 0;
    const int Gp = (G + 3) & ~3;
    const int srow = T.e >= 0 ? A.perm[T.m0 + src] / A.top_k : T.m0 + src;
    const rsrc_t gres = buf_rsrc(A.xg, (uint32_t)((size_t)A.rows * Gp * 4));
    constexpr int kQ = 3;  // quads of groups per thread per batch: 48 groups (d_model 3072) in one batch
    for (int u0 = 0; 16 * u0 < G; u0 += kQ) {
      u32x4_t v[kQ];
#pragma unroll
      for (int u = 0; u < kQ; ++u)
        v[u] = bld16(gres, (uint32_t)((srow * Gp + 4 * ((tid >> 6) + 4 * (u0 + u))) * 4), 0);
#pragma unroll
      for (int u = 0; u < kQ; ++u) {
        const int g = 4 * ((tid >> 6) + 4 * (u0 + u));
        if (g < G) {  // wave-uniform
#pragma unroll
          for (int c = 0; c < 4; ++c)
            S.xgL[(g + c) * 64 + r] = g + c < G ? __uint_as_float(v[u][c]) : 0.0f;  // zeros up to a multiple of 4
        }
      }
    }
  }
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
    // The bias term sum_g (b_g - 128 s_g) X_g of four consecutive groups is one fp32
    // 16x16x4 matrix product per row block and matrix: lane 16k + n collects column n's
    // (b - 128 s) of the k-th group of the four in bsel (each group writes its own lane
    // row), and the A operand is the group sums X of those groups from LDS (zero past G).
    // Ring slot j holds group g0 + j with g0 a multiple of kRing, so j % 4 is the group's
    // place among its four.
    static_assert(kRing % 4 == 0, "a ring pass covers whole sets of four groups");
    float bsel[2] = {0.0f, 0.0f};
    auto bias4 = [&](int gq) __attribute__((always_inline)) {
  #pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        const float a4 = S.xgL[(gq + (lane >> 4)) * 64 + 16 * mb + (lane & 15)];
  #pragma unroll
        for (int m = 0; m < 2; ++m) acc[mb][m] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4, bsel[m], acc[mb][m], 0, 0, 0);
      }
      bsel[0] = bsel[1] = 0.0f;  // lanes of groups past G stay zero in a last partial set
    };

    // One stage = SG K groups from LDS buffer (j0 / SG) & 1 and weight slots j0.. j0 + SG - 1:
    // per group the codes of its slot become MFMA operands and the slot is refilled with
    // group g + kRing; after the stage's MFMAs the next stage is staged into the other
    // buffer from the activation ring and its slots refilled SG stages ahead (loads past
    // the last group are clamped to it and never used). The steady-state loop is
    // straight-line code over kRing groups, so every ring slot keeps its own registers
    // and no wait covers a load younger than the one it needs.
    const NibK nk;
    auto stage = [&](auto jc, int g) __attribute__((always_inline)) {
      constexpr int j0 = decltype(jc)::value;
      constexpr int buf = (j0 / SG) & 1;
      static_for<SG>([&](auto pc) __attribute__((always_inline)) {
        constexpr int p = decltype(pc)::value;
        constexpr int j = j0 + p;
        bf16x8_t bfr[2][2];
        float s[2], bb[2];
        const u32x4_t cw = B.codes(ic<j>{});
        const u32x2_t sbw = B.scales(ic<j>{});
  #pragma unroll
        for (int m = 0; m < 2; ++m) {
          bfr[m][0] = codes_bf16(cw[2 * m], nk);
          bfr[m][1] = codes_bf16(cw[2 * m + 1], nk);
          s[m] = bf16_lo(sbw[m]);
          bb[m] = fmaf(-128.0f, s[m], bf16_hi(sbw[m]));  // b - 128 s
          bsel[m] = (lane >> 4) == (j & 3) ? bb[m] : bsel[m];
        }
        B.load(ic<j>{}, wres, min(g + p + kRing, G - 1));
  #pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
          const int ao = buf * kBuf + (16 * mb + (lane & 15)) * kStride + p * 64 + 8 * (lane >> 4);
          const bf16x8_t a0 = lds_frag<bf16x8_t>(&Xs[ao]);
          const bf16x8_t a1 = lds_frag<bf16x8_t>(&Xs[ao + 32]);
          f32x4_t t[2];
  #pragma unroll
          for (int m = 0; m < 2; ++m) t[m] = mfma(a1, bfr[m][1], mfma(a0, bfr[m][0], f32x4_t{0.f, 0.f, 0.f, 0.f}));
          if (LO) {
            const bf16x8_t l0 = lds_frag<bf16x8_t>(&Xls[ao]);
            const bf16x8_t l1 = lds_frag<bf16x8_t>(&Xls[ao + 32]);
  #pragma unroll
            for (int m = 0; m < 2; ++m) t[m] = mfma(l1, bfr[m][1], mfma(l0, bfr[m][0], t[m]));
          }
  #pragma unroll
          for (int m = 0; m < 2; ++m)
  #pragma unroll
            for (int i = 0; i < 4; ++i) acc[mb][m][i] = fmaf(s[m], t[m][i], acc[mb][m][i]);
        }
        if constexpr ((j & 3) == 3) bias4(g + p - 3);
      });
      // the next stage into the other buffer (its readers passed the last barrier)
      static_for<SG>([&](auto pc) __attribute__((always_inline)) {
        constexpr int p = decltype(pc)::value;
        constexpr int slot = (j0 + SG + p) % RA;
        astore(ic<slot>{}, buf ^ 1);
        aload(ic<slot>{}, min(g + SG + p + RA, G - 1));
      });
      __syncthreads();
    };
    int g0 = 0;
    for (; g0 + kRing <= G; g0 += kRing)
      static_for<kRing / SG>([&](auto sc) __attribute__((always_inline)) {
        constexpr int st = decltype(sc)::value;
        stage(ic<st * SG>{}, g0 + st * SG);
      });
    // the last G % kRing groups (a multiple of SG)
    static_for<kRing / SG - 1>([&](auto sc) __attribute__((always_inline)) {
      constexpr int st = decltype(sc)::value;
      if (g0 + st * SG < G) stage(ic<st * SG>{}, g0 + st * SG);
    });
    if (G & 3) bias4(G & ~3);  // the last partial set of four


    // GeGLU epilogue: lane holds rows 16mb + 4*(lane/16) + i, d_ff column fc*64 + 16*wave + lane%16.
    // h goes out as fp16, scaled per (row, 64-column block) by the power of two that brings
    // the block's largest |h| into [2^14, 2^15); the scale goes out beside it (the down
    // kernel brings a row's blocks to one scale as it stages them).
    uint16_t* Hh = shared ? A.Hh + (size_t)A.rows * A.top_k * A.f : A.Hh;
    float* hbs = shared ? A.hbs + (size_t)A.rows * A.top_k * (A.f / 64) : A.hbs;
    const int F = T.F, nG = F / 64;
    float hv[NMB][4];
  #pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mb + 4 * (lane >> 4) + i;
        hv[mb][i] = r < T.mrows ? gelu_tanh(acc[mb][0][i]) * acc[mb][1][i] : 0.0f;
        // max |h| over the 16 lanes holding this row: one DPP row (VALU, no LDS round trips)
        const float mx = row16_max(fabsf(hv[mb][i]));
        if ((lane & 15) == 0) hmL[wave][r] = mx;
      }
    __syncthreads();
    if (tid < 64) {
      const float sc = row_scale(fmaxf(fmaxf(hmL[0][tid], hmL[1][tid]), fmaxf(hmL[2][tid], hmL[3][tid])));
      S.hsL[tid] = sc;
      if (tid < T.mrows) hbs[(size_t)(T.m0 + tid) * nG + fc] = sc;
    }
    __syncthreads();
  #pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      const f32x4_t sc = *reinterpret_cast<const f32x4_t*>(&S.hsL[16 * mb + 4 * (lane >> 4)]);
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mb + 4 * (lane >> 4) + i;
        if (r < T.mrows) Hh[(size_t)(T.m0 + r) * F + fc * 64 + 16 * wave + (lane & 15)] = f16_bits(hv[mb][i] * sc[i]);
      }
    }

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
    // bf16 activations with an even group count stage two groups per barrier
    if (sizeof(XT) == 2 && (A.d / kGroup) % 2 == 0)
      gateup_tile<XT, sizeof(XT) == 2 ? 2 : 1>(A, x, T, fc, shared, S);
    else
      gateup_tile<XT, 1>(A, x, T, fc, shared, S);
    __syncthreads();  // the next item reuses the LDS
  }
}

// ---------------------------------------------------------------- down

struct DownSmem {
  __attribute__((aligned(16))) uint16_t Hl[2][64 * kLdsStride];
  float rowinv[64];
  __attribute__((aligned(16))) float agL[2][64];  // per-row sums of the staged H group
};

// One work item = (64-row tile, four blocks of 64 output columns, 4 np .. 4 np + 3).
// Wave w owns output columns [16w, +16) of every block for every row of the tile, so
// one staged H tile feeds four times the columns, and a 128-row chunk's items fit the
// chip's resident workgroups in one round. The weights come in two rings of two blocks
// each, two groups deep. Blocks past the last one repeat it and are not stored.
constexpr int kDownBlocks = 4;
constexpr int kDownRing = 2;  // weight groups in flight per ring
__device__ __forceinline__ void down_tile(const PrefillArgs& A, const MTile& T, int np, bool shared, int part,
                                          DownSmem& S) {
  constexpr int RA = 2;  // H groups in flight
  auto& Hl = S.Hl;
  auto& rowinv = S.rowinv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int F = T.F, G = F / kGroup;
  // K groups [gb, ge) of this item: all of a routed expert's, part `part` of the shared expert's
  const int gp = (G + kSharedDownParts - 1) / kSharedDownParts;
  const int gb = shared ? min(G, part * gp) : 0, ge = shared ? min(G, gb + gp) : G;
  const int nmb = (T.mrows + 15) >> 4;
  const int P = A.rows * A.top_k;
  const uint16_t* Hh = shared ? A.Hh + (size_t)P * A.f : A.Hh;
  const float* hbs = shared ? A.hbs + (size_t)P * (A.f / 64) : A.hbs;

  const int wrow = 16 * wave + (lane & 15);
  const int nblk = A.d / 64;
  static_assert(kDownBlocks == 4, "two weight rings of two blocks each");
  static_assert(4 % kDownRing == 0, "the unrolled steps cover whole ring passes");
  int nbm[kDownBlocks];
#pragma unroll
  for (int m = 0; m < kDownBlocks; ++m) nbm[m] = min(kDownBlocks * np + m, nblk - 1);
  rsrc_t wres[2];
  BRingT<kDownRing> B[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const uint32_t mstride = (uint32_t)(nbm[2 * p + 1] - nbm[2 * p]) * G * kTile4;  // 0 for a repeated block
    wres[p] = buf_rsrc(uniform_ptr(T.blob) + 2 * m4_bytes(F, A.d) + (uint64_t)nbm[2 * p] * G * kTile4,
                       mstride + (uint32_t)G * kTile4);
    B[p].init(wrow, lane, mstride);
  }

  // H staging: thread -> tile row tid/4, 16 halfs at column (tid%4)*16; rows past
  // the tile's end repeat its first row (see the gate/up kernel)
  const int hr = tid >> 2, hq = tid & 3;
  const int hrow = T.m0 + (hr < T.mrows ? hr : 0);
  const rsrc_t hres = buf_rsrc(Hh, (uint32_t)((size_t)(shared ? A.rows : P) * F * sizeof(uint16_t)));
  const uint32_t hvo = (uint32_t)(((size_t)hrow * F + hq * 16) * sizeof(uint16_t));
  // the row's scale in this item: the smallest of its blocks' scales over [gb, ge) (that
  // of its largest block), as the exponent field of the power of two; each staged block
  // is brought to it by an exact power-of-two product (at most 1), and the outputs are
  // divided by it at the end
  const rsrc_t sres = buf_rsrc(hbs, (uint32_t)((size_t)(shared ? A.rows : P) * G * sizeof(float)));
  const uint32_t svo = (uint32_t)((size_t)hrow * G * sizeof(float));
  // (the first 16 groups' scales in one batch of loads, in flight with the prologue's)
  uint32_t emin = 255u;
  uint32_t sv[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) sv[j] = bld4(sres, svo + (uint32_t)min(gb + j, ge - 1) * 4u, 0);
  for (int g = gb + 16; g < ge; ++g) emin = min(emin, (bld4(sres, svo + (uint32_t)g * 4u, 0) >> 23) & 0xffu);
  u32x4_t ha[RA][2];
  uint32_t hs[RA];
  auto aload = [&](auto sc, int g) __attribute__((always_inline)) {
    constexpr int slot = decltype(sc)::value;
    const uint32_t so = (uint32_t)(g * kGroup * sizeof(uint16_t));
    ha[slot][0] = bld16(hres, hvo, so);
    ha[slot][1] = bld16(hres, hvo + 16, so);
    hs[slot] = bld4(sres, svo + (uint32_t)g * 4u, 0);
  };
  // the staging threads also add up each row's group (dot products against fp16 (1, 1)
  // pairs, the four threads of a row summed by DPP) for the bias term of the epilogue
  auto astore = [&](auto sc, int buf) __attribute__((always_inline)) {
    constexpr int slot = decltype(sc)::value;
    // 2^(emin - e) for this block's exponent e: the fp16 product rounds only below the
    // fp16 normal range (values 2^-28 of the row's largest or smaller)
    const uint32_t m1 = f16_bits(ldexpf(1.0f, (int)emin - (int)((hs[slot] >> 23) & 0xffu)));
    const f16x2_t m2 = __builtin_bit_cast(f16x2_t, m1 | (m1 << 16));
    u32x4_t hv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        hv[h][c] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, (uint32_t)ha[slot][h][c]) * m2);
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(&Hl[buf][hr * kLdsStride + hq * 16]);
    dst[0] = hv[0];
    dst[1] = hv[1];
    float v = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t w = hv[h][c];  // a bit_cast of the vector element itself reads element 0
        v = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, w), __builtin_bit_cast(f16x2_t, 0x3C003C00u), v, false);
      }
    v = dpp_add<0xB1, 0xf>(v);  // the four threads of a row are one quad
    v = dpp_add<0x4E, 0xf>(v);
    if (hq == 0) S.agL[buf][hr] = v;
  };
  float* out = shared ? A.shared_out + (size_t)part * A.rows * A.d : A.expert_out;
  if (ge <= gb) {  // an empty part (d_ff_shared under kSharedDownParts groups): zeros
    if (tid < 64)
      for (int m = 0; m < kDownBlocks && kDownBlocks * np + m < nblk; ++m)
        for (int r = 0; r < T.mrows; ++r) out[(size_t)(T.m0 + r) * A.d + nbm[m] * 64 + tid] = 0.0f;
    return;
  }
  // prologue: the loads in the order the steady state issues them (weights of group
  // j, then activations of group j + 1), so the wait counts agree on entry
  aload(ic<0>{}, gb);
  static_for<RA>([&](auto jc) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    if constexpr (j < kDownRing) {
      B[0].load(jc, wres[0], min(gb + j, ge - 1));
      B[1].load(jc, wres[1], min(gb + j, ge - 1));
    }
    if constexpr (j + 1 < RA) aload(ic<j + 1>{}, min(gb + j + 1, ge - 1));
    if constexpr (j + 1 == RA) {
#pragma unroll
      for (int t = 0; t < 16; ++t) emin = min(emin, (sv[t] >> 23) & 0xffu);
      if (hq == 0) rowinv[hr] = 1.0f / __uint_as_float(emin << 23);  // exact: a power of two
      astore(ic<0>{}, 0);
      aload(ic<0>{}, min(gb + RA, ge - 1));
    }
  });
  __syncthreads();

  f32x4_t acc[4][kDownBlocks];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int m = 0; m < kDownBlocks; ++m) zero_acc(acc[mb][m]);

  // one K group, as in the gate/up kernel (H slot j of RA, weight slot j % kDownRing);
  // one ring's two blocks at a time, so only their operands are live
  const NibKT<0x64006400u> nk;
  auto step = [&](auto jc, int g) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    constexpr int buf = j & 1;
    constexpr int ws = j % kDownRing;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      f16x8_t b0[2], b1[2];
      float s[2], bp[2];
      const u32x4_t cw = B[p].codes(ic<ws>{});
      const u32x2_t sbw = B[p].scales(ic<ws>{});
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        b0[h] = codes_f16(cw[2 * h], nk);
        b1[h] = codes_f16(cw[2 * h + 1], nk);
        s[h] = bf16_lo(sbw[h]);
        bp[h] = fmaf(-1024.0f, s[h], bf16_hi(sbw[h]));  // b - 1024 s (exact)
      }
      B[p].load(ic<ws>{}, wres[p], min(g + kDownRing, ge - 1));
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        if (mb < nmb) {
          const int ao = (16 * mb + (lane & 15)) * kLdsStride + 8 * (lane >> 4);
          const f16x8_t a0 = lds_frag<f16x8_t>(&Hl[buf][ao]);
          const f16x8_t a1 = lds_frag<f16x8_t>(&Hl[buf][ao + 32]);
          const f32x4_t ag = *reinterpret_cast<const f32x4_t*>(&S.agL[buf][16 * mb + 4 * (lane >> 4)]);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const f32x4_t t = mfma(a1, b1[h], mfma(a0, b0[h], f32x4_t{0.f, 0.f, 0.f, 0.f}));
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[mb][2 * p + h][i] = fmaf(s[h], t[i], fmaf(bp[h], ag[i], acc[mb][2 * p + h][i]));
          }
        }
      }
    }
    astore(ic<(j + 1) % RA>{}, buf ^ 1);
    aload(ic<(j + 1) % RA>{}, min(g + 1 + RA, ge - 1));
    __syncthreads();
  };
  int g0 = gb;
  static_assert(RA == 2 && kDownRing == 2, "the loop below is unrolled over two H and weight slots");
  for (; g0 + RA <= ge; g0 += RA) {
    step(ic<0>{}, g0);
    step(ic<1>{}, g0 + 1);
  }
  if (g0 < ge) step(ic<0>{}, g0);
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
  // the shared expert's items: (row tile, K part) pairs x column blocks
  const int nsp = A.shared_mtiles * kSharedDownParts;
  const int ns = xcd_blocks(nsp, nc);
  const int n = ns + xcd_blocks(nrt, nc);
  for (int item = blockIdx.x; item < n; item += gridDim.x) {
    const bool shared = item < ns;
    int mt, nb, part = 0;
    MTile T;
    if (shared) {
      xcd_item(item, nsp, nc, mt, nb);
      if (mt >= nsp) continue;
      part = mt % kSharedDownParts;
      shared_tile(A, mt / kSharedDownParts, T);
    } else {
      xcd_item(item - ns, nrt, nc, mt, nb);
      if (mt >= nrt || !tile_at(A, M, mt, T)) continue;
    }
    down_tile(A, T, nb, shared, part, S);
    __syncthreads();  // the next item reuses the LDS
  }
}

}  // namespace qmoe
