// Device pieces shared by the two forms of the continuous-gate backward (one
// decode step; the training-time forward of one sequence): the transpose of
// RoPE, the gate-key projection of pooled block statistics on MFMA, and
// weight gradients as fixed-order sums of outer products on MFMA.
#pragma once
#include "sas_device.h"

namespace sas {

constexpr float kInvSqrtDg = 0.08838834764831845f;  // 1/sqrt(128)

__device__ __forceinline__ bf16x8 to_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// the transpose of the rotate-half RoPE rotation at one pair (i, i+64)
__device__ __forceinline__ void rope_back(float da, float db, float c, float s, float &ga, float &gb) {
  ga = da * c + db * s;
  gb = db * c - da * s;
}

// ---------------------------------------------------------------- gate-key projection of pooled statistics
// U^T = W_k[kvh] P^T for kChainBlocks blocks' pooled statistics P (rows of
// 384: max, min, mean), 256 threads.  Wave w owns the projection rows
// 32w .. 32w+31; lane l feeds block l%16 and inputs 32ks + 8(l/16) .. +7.
// The max and min inputs are bf16 values; the mean inputs are split into bf16
// high and low parts (about 16 significant bits).
constexpr int kPoolPitch = 3 * kHeadDim + 4;  // LDS row of pooled statistics (floats), staggered banks
constexpr int kUkPitch = kGateDim + 4;

// W_k A operands of this wave's 32 rows (row 32w + 16mt + l%16, inputs
// 32ks + 8(l/16) .. +7), w_k laid out [Hkv][128][384]
__device__ __forceinline__ void load_wk_rows(const uint16_t *w_k, int kvh, u32x4 (&wk)[2][12]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint16_t *wkb = w_k + ((int64_t)kvh * kGateDim + 32 * wave + (lane & 15)) * 3 * kHeadDim + 8 * (lane >> 4);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) wk[mt][ks] = ld16(wkb + (int64_t)16 * mt * 3 * kHeadDim + 32 * ks);
}

// uk[b][r] = row r of W_k applied to pooled[b] for the 16 blocks b (rows of
// blocks not filled hold stale values; the caller reads only its own)
template <int kRows>
__device__ __forceinline__ void project_pooled(const u32x4 (&wk)[2][12], const float (*pooled)[kPoolPitch],
                                               float (*uk)[kUkPitch]) {
  static_assert(kRows == 16, "one MFMA column per block");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  const float *pb = &pooled[lane & 15][8 * (lane >> 4)];
#pragma unroll
  for (int ks = 0; ks < 12; ++ks) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = pb[32 * ks + e];
    const u32x4 h = {pack_bf16_rne(x[0], x[1]), pack_bf16_rne(x[2], x[3]), pack_bf16_rne(x[4], x[5]),
                     pack_bf16_rne(x[6], x[7])};
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(to_bf16x8(wk[mt][ks]), to_bf16x8(h), acc[mt], 0, 0, 0);
    if (ks >= 8) {
      float lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) lo[e] = x[e] - ((e & 1) ? bf16_hi(h[e >> 1]) : bf16_lo(h[e >> 1]));
      const u32x4 l = {pack_bf16_rne(lo[0], lo[1]), pack_bf16_rne(lo[2], lo[3]), pack_bf16_rne(lo[4], lo[5]),
                       pack_bf16_rne(lo[6], lo[7])};
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(to_bf16x8(wk[mt][ks]), to_bf16x8(l), acc[mt], 0, 0, 0);
    }
  }
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) uk[lane & 15][32 * wave + 16 * mt + 4 * (lane >> 4) + r] = acc[mt][r];
}

// ---------------------------------------------------------------- sums of outer products
// acc = sum over rows n in [n_lo, n_hi) of A(n, 64-wide column slice) (x)
// B(n, 64-wide column slice) for one 64 x 64 tile.  The fp32 operands are
// split into bf16 high and low parts and summed as hi*hi + hi*lo + lo*hi on
// v_mfma_f32_16x16x32_bf16 (the dropped lo*lo term is ~2^-16 relative; the
// split itself keeps ~16 significant bits).  Rows go through LDS 32 at a
// time, already split and transposed (column-major, 8 rows per 16 bytes,
// a 40-element pitch so that the operand reads are conflict-free), the next
// 32 fetched into registers while the current ones are summed (fetching
// further ahead measured slower): thread t fetches rows 8(t/64) .. +7 of
// column t%64.  Wave w owns the 32 x 32 quadrant (rows 32(w/2), columns
// 32(w%2)) as 2 x 2 MFMA tiles; lane l feeds column l%16 of its tile and the
// step's rows 8(l/16) .. +7 to both operands.  The rows are taken in order
// (deterministic).  256 threads.
constexpr int kOsPitch = 40;  // bf16 elements per LDS column of 32 rows
struct OuterLds {
  uint16_t ah[64][kOsPitch], al[64][kOsPitch], bh[64][kOsPitch], bl[64][kOsPitch];
};

template <typename FA, typename FB>
__device__ void outer_sum_tile(FA fa, FB fb, int n_lo, int n_hi, f32x4 (&acc)[2][2], OuterLds &ls) {
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int wm = wave >> 1, wn = wave & 1, g = lane >> 4, c16 = lane & 15;
  const int col = t & 63, rg = t >> 6;  // fetch: column, group of 8 rows
  float ra[8], rb[8];
  auto fetch = [&](int n0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int n = n0 + 8 * rg + e;
      ra[e] = n < n_hi ? fa(n, col) : 0.f;
      rb[e] = n < n_hi ? fb(n, col) : 0.f;
    }
  };
  auto split = [&](const float (&x)[8], uint16_t *hi, uint16_t *lo) {
    u32x4 h, l;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t hp = pack_bf16_rne(x[2 * q], x[2 * q + 1]);
      h[q] = hp;
      l[q] = pack_bf16_rne(x[2 * q] - bf16_lo(hp), x[2 * q + 1] - bf16_hi(hp));
    }
    *reinterpret_cast<u32x4 *>(hi) = h;
    *reinterpret_cast<u32x4 *>(lo) = l;
  };
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (n_lo < n_hi) fetch(n_lo);
  for (int n0 = n_lo; n0 < n_hi; n0 += 32) {
    lds_barrier();
    split(ra, &ls.ah[col][8 * rg], &ls.al[col][8 * rg]);
    split(rb, &ls.bh[col][8 * rg], &ls.bl[col][8 * rg]);
    lds_barrier();
    if (n0 + 32 < n_hi) fetch(n0 + 32);
    bf16x8 ah[2], al[2], bh[2], bl[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      ah[i] = to_bf16x8(*reinterpret_cast<const u32x4 *>(&ls.ah[32 * wm + 16 * i + c16][8 * g]));
      al[i] = to_bf16x8(*reinterpret_cast<const u32x4 *>(&ls.al[32 * wm + 16 * i + c16][8 * g]));
      bh[i] = to_bf16x8(*reinterpret_cast<const u32x4 *>(&ls.bh[32 * wn + 16 * i + c16][8 * g]));
      bl[i] = to_bf16x8(*reinterpret_cast<const u32x4 *>(&ls.bl[32 * wn + 16 * i + c16][8 * g]));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], bh[j], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], bl[j], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[i], bh[j], acc[i][j], 0, 0, 0);
      }
  }
}

// The same sum for a 128 x 128 tile: acc(m, c) = sum over rows n of
// fa4(n, m)[k] * fb4(n, c)[k'] for the columns m + k, c + k' (fa4 / fb4 give
// four adjacent columns, m and c multiples of 4).  Wave w owns rows
// 64(w/2) .. +63 and columns 64(w%2) .. +63 (4 x 4 MFMA tiles: 48 MFMAs per
// 32 rows, four times the 64 x 64 tile's MFMAs for each LDS round); thread
// t fetches rows 4(t/32) .. +3 of the 32 and columns 4(t%32) .. +3.
// kExactB: fb's values are bf16 (their low parts are zero), so the
// high(a) x low(b) products are skipped.
struct OuterLds128 {
  uint16_t ah[128][kOsPitch], al[128][kOsPitch], bh[128][kOsPitch], bl[128][kOsPitch];
};

template <bool kExactB, typename FA4, typename FB4>
__device__ void outer_sum_tile128(FA4 fa4, FB4 fb4, int n_lo, int n_hi, f32x4 (&acc)[4][4], OuterLds128 &ls) {
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int wm = wave >> 1, wn = wave & 1, g = lane >> 4, c16 = lane & 15;
  const int c4 = 4 * (t & 31), rg = t >> 5;
  f32x4 ra[4], rb[4];
  auto fetch = [&](int n0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = n0 + 4 * rg + r;
      ra[r] = n < n_hi ? fa4(n, c4) : f32x4{0.f, 0.f, 0.f, 0.f};
      rb[r] = n < n_hi ? fb4(n, c4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  // column c4 + k, rows 4rg .. +3: bf16 high parts and (if wanted) the
  // bf16 rounding of what they leave
  auto split = [&](const f32x4 (&x)[4], uint16_t (*hi)[kOsPitch], uint16_t (*lo)[kOsPitch], bool low_parts) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t h0 = pack_bf16_rne(x[0][k], x[1][k]), h1 = pack_bf16_rne(x[2][k], x[3][k]);
      *reinterpret_cast<u32x2 *>(&hi[c4 + k][4 * rg]) = u32x2{h0, h1};
      if (low_parts)
        *reinterpret_cast<u32x2 *>(&lo[c4 + k][4 * rg]) =
            u32x2{pack_bf16_rne(x[0][k] - bf16_lo(h0), x[1][k] - bf16_hi(h0)),
                  pack_bf16_rne(x[2][k] - bf16_lo(h1), x[3][k] - bf16_hi(h1))};
    }
  };
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (n_lo < n_hi) fetch(n_lo);
  for (int n0 = n_lo; n0 < n_hi; n0 += 32) {
    lds_barrier();
    split(ra, ls.ah, ls.al, true);
    split(rb, ls.bh, ls.bl, !kExactB);
    lds_barrier();
    if (n0 + 32 < n_hi) fetch(n0 + 32);
    bf16x8 ah[4], al[4], bh[4], bl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ah[i] = to_bf16x8(*reinterpret_cast<const u32x4 *>(&ls.ah[64 * wm + 16 * i + c16][8 * g]));
      al[i] = to_bf16x8(*reinterpret_cast<const u32x4 *>(&ls.al[64 * wm + 16 * i + c16][8 * g]));
      bh[i] = to_bf16x8(*reinterpret_cast<const u32x4 *>(&ls.bh[64 * wn + 16 * i + c16][8 * g]));
      if (!kExactB) bl[i] = to_bf16x8(*reinterpret_cast<const u32x4 *>(&ls.bl[64 * wn + 16 * i + c16][8 * g]));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], bh[j], acc[i][j], 0, 0, 0);
        if (!kExactB) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], bl[j], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[i], bh[j], acc[i][j], 0, 0, 0);
      }
  }
}

// writes a tile from outer_sum_tile128 to a dense 128 x 128 buffer: lane l
// of wave w holds rows 64(w/2) + 16i + 4(l/16) + r, column 64(w%2) + 16j + l%16
__device__ __forceinline__ void store_tile128(const f32x4 (&acc)[4][4], float *dst) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        dst[(64 * wm + 16 * i + 4 * (lane >> 4) + r) * 128 + 64 * wn + 16 * j + (lane & 15)] = acc[i][j][r];
}

// writes a tile from outer_sum_tile: lane l of wave w holds rows
// 32(w/2) + 16i + 4(l/16) + r, column 32(w%2) + 16j + l%16
__device__ __forceinline__ void store_tile(const f32x4 (&acc)[2][2], float *dst, int64_t row_stride) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        dst[(int64_t)(32 * wm + 16 * i + 4 * (lane >> 4) + r) * row_stride + 32 * wn + 16 * j + (lane & 15)] =
            acc[i][j][r];
}

// dst[e] = sum over parts of src[part * part_stride + e] for the 4096 elements
// of a 64 x 64 tile, parts in order; dst row r at dst + r * row_stride.
// 256 threads, thread t owns elements 4(t + 256q) .. +3.
__device__ __forceinline__ void sum_tile_parts(const float *src, int parts, int64_t part_stride, float *dst,
                                               int64_t row_stride) {
  f32x4 acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int part = 0; part < parts; ++part)
      acc[q] += *reinterpret_cast<const f32x4 *>(src + part * part_stride + 4 * (threadIdx.x + 256 * q));
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = 4 * (threadIdx.x + 256 * q);
    float *d = dst + (int64_t)(e >> 6) * row_stride + (e & 63);
#pragma unroll
    for (int v = 0; v < 4; ++v) d[v] = acc[q][v];
  }
}

}  // namespace sas
