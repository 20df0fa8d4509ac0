// Exact Top-K of one row of order-preserving score keys by one wave, shared
// by the decode selection and the training-time forward's selection.
#pragma once
#include "sas_device.h"

namespace sas {

// Inclusive prefix sum over the 64 lanes of a wave (DPP row shifts, then the
// row broadcasts of lanes 15 and 31).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Exact Top-K of the n candidate keys keys[0 .. n) of one (sequence or
// position, KV head) under (score descending, index ascending), by one wave.
// keys: LDS, 16-byte aligned, readable up to max(n, 512) entries (keys are
// > 0; entries past n are ignored); hist: this wave's 256-entry LDS
// histogram.  Radix select over 8-bit digits with a wave-private histogram
// and DPP prefix sums: the threshold key T is found digit by digit, most
// significant first; the Top-K is every key > T and the krem lowest-index
// keys equal to T.  Lane l sweeps keys [512k + 8l, 512k + 8l + 8); the first
// 512 stay in registers across the passes.
struct WaveTopK {
  const uint32_t *keys;
  int n, k_eff, lane;
  uint32_t k0[8];  // keys 8l .. 8l+7 (0 past the candidates: keys are > 0)
  uint32_t prefix, mask, T, krem;
  int shift;       // digit of the next pass; < 0 when T is final

  __device__ __forceinline__ void init(const uint32_t *keys_, int n_, int k_eff_) {
    keys = keys_;
    n = n_;
    k_eff = k_eff_;
    lane = threadIdx.x & 63;
    const u32x4 a = *reinterpret_cast<const u32x4 *>(&keys[8 * lane]);
    const u32x4 b = *reinterpret_cast<const u32x4 *>(&keys[8 * lane + 4]);
    const uint32_t r[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) k0[e] = 8 * lane + e < n ? r[e] : 0u;
    prefix = mask = 0;
    T = 0;  // k_eff >= n: every candidate (all keys are > 0)
    krem = 0;
    shift = -8;
    if (k_eff > 0 && k_eff < n) {
      krem = (uint32_t)k_eff;
      shift = 24;
    }
  }

  __device__ __forceinline__ uint32_t key_at(int c0, int e) const {  // key c0 + e of this lane's sweep
    return c0 == 8 * lane ? k0[e] : (c0 + e < n ? keys[c0 + e] : 0u);
  }

  // The radix passes (digits 24, 16, 8, 0; none when shift < 0).
  __device__ __forceinline__ void passes(uint32_t *hist) {
    for (int sh = 24; sh >= 0; sh -= 8) {
      if (sh > shift) continue;  // T is final without passes (shift < 0)
      *reinterpret_cast<u32x4 *>(&hist[4 * lane]) = u32x4{0, 0, 0, 0};
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (k0[e] != 0u && (k0[e] & mask) == prefix) atomicAdd(&hist[(k0[e] >> sh) & 255u], 1u);
      for (int c0 = 8 * lane + 512; c0 < n; c0 += 512) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t k = key_at(c0, e);
          if (k != 0u && (k & mask) == prefix) atomicAdd(&hist[(k >> sh) & 255u], 1u);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // lane l owns digits 255-4l .. 252-4l (descending)
      const u32x4 h4 = *reinterpret_cast<const u32x4 *>(&hist[252 - 4 * lane]);
      const uint32_t cnt[4] = {h4.w, h4.z, h4.y, h4.x};
      const uint32_t tot = cnt[0] + cnt[1] + cnt[2] + cnt[3];
      uint32_t run = wave_incl_scan(tot) - tot;  // keys in higher digits
      int found_e = -1;
      uint32_t found_krem = 0, found_cnt = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (found_e < 0 && run < krem && run + cnt[e] >= krem) {
          found_e = e;
          found_krem = krem - run;
          found_cnt = cnt[e];
        }
        run += cnt[e];
      }
      const unsigned long long who = __ballot(found_e >= 0);
      const int leader = (int)__builtin_ctzll(who);  // exactly one lane finds the digit
      const uint32_t d = 255u - (uint32_t)(4 * leader + __builtin_amdgcn_readlane(found_e, leader));
      krem = (uint32_t)__builtin_amdgcn_readlane((int)found_krem, leader);
      const uint32_t bin_cnt = (uint32_t)__builtin_amdgcn_readlane((int)found_cnt, leader);
      prefix |= d << sh;
      mask |= 0xFFu << sh;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      if (bin_cnt == krem) {  // the whole bin is taken: every key >= prefix
        // prefix == 0 (all digits so far 0) only when every non-zero key left
        // lies in this bin, which holds when padding (key 0) follows fewer
        // non-zero keys than n: then every non-zero key is taken (keys > 0)
        T = prefix ? prefix - 1u : 0u;
        krem = 0;
        shift = -8;
        break;
      }
      T = prefix;
      shift = sh - 8;
    }
  }

  // Calls emit(pos, c, key) for the keys > Tt and the kr lowest-index keys
  // equal to Tt, those at most hi (>= Tt), in ascending c, pos = their rank
  // among them.
  template <class Emit>
  __device__ __forceinline__ void sweep(uint32_t Tt, uint32_t kr, uint32_t hi, Emit emit) const {
    uint32_t pos_base = 0, eq_base = 0;
    for (int c0 = 0; c0 < n; c0 += 512) {
      const int cl = c0 + 8 * lane;
      uint32_t kk[8];
      uint32_t n_eq = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kk[e] = key_at(cl, e);
        n_eq += (kr > 0 && kk[e] == Tt);
      }
      const uint32_t eq_incl = wave_incl_scan(n_eq);
      uint32_t eq_rank = eq_base + eq_incl - n_eq;  // equal keys before this lane's
      uint32_t take_mask = 0, n_take = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bool take = kk[e] > Tt && kk[e] <= hi;
        if (kr > 0 && kk[e] == Tt) take = eq_rank++ < kr;
        take_mask |= (uint32_t)take << e;
        n_take += take;
      }
      const uint32_t take_incl = wave_incl_scan(n_take);
      uint32_t pos = pos_base + take_incl - n_take;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (take_mask >> e & 1u) emit(pos++, cl + e, kk[e]);
      pos_base += (uint32_t)__builtin_amdgcn_readlane((int)take_incl, 63);
      eq_base += (uint32_t)__builtin_amdgcn_readlane((int)eq_incl, 63);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
};

// The whole Top-K: calls emit(pos, c, key) for the k_eff chosen candidates
// c, pos = 0 .. k_eff-1 in ascending c (WaveTopK).
template <class Emit>
__device__ __forceinline__ void wave_select_emit(const uint32_t *keys, int n, int k_eff, uint32_t *hist, Emit emit) {
  WaveTopK tk;
  tk.init(keys, n, k_eff);
  tk.passes(hist);
  if (k_eff > 0) tk.sweep(tk.T, tk.krem, 0xFFFFFFFFu, emit);
}

// Writes the selection of one (sequence or position, KV head): the k_eff
// best candidates (wave_select_emit) in ascending block order, then the
// local block n; padding -1 up to n_sel; gates (nullable) = sigmoid(score)
// for the chosen historical blocks, 1 for the local block, 0 padding;
// *cnt = k_eff + 1.  hist afterwards holds the compacted selection
// (n_sel <= 256).
__device__ __forceinline__ void wave_select(const uint32_t *keys, int n, int k_eff, int n_sel, uint32_t *hist,
                                            int32_t *sel, float *gates, int32_t *cnt_out) {
  const int lane = threadIdx.x & 63;
  wave_select_emit(keys, n, k_eff, hist, [&](uint32_t pos, int c, uint32_t) { hist[pos] = (uint32_t)c; });
  for (int i = lane; i < n_sel; i += 64) {
    int32_t c;
    float g;
    if (i < k_eff) {
      c = (int32_t)hist[i];
      g = 1.0f / (1.0f + __expf(-key_score(keys[c])));
    } else {
      c = i == k_eff ? n : -1;
      g = i == k_eff ? 1.0f : 0.0f;
    }
    sel[i] = c;
    if (gates) gates[i] = g;
  }
  if (lane == 0) *cnt_out = k_eff + 1;
}

}  // namespace sas

