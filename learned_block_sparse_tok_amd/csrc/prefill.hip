// Training-time forward: every position of one sequence attends its own
// block selection.
//
// SAS selects KV blocks for each query and trains with a Top-K of 31
// historical 64-token blocks on 32,768-token sequences ("Tencent released
// Simple-Attention-Sparsification ...", aigc.news; "Tencent Hunyuan
// open-sources SAS ...": per-query block selection).  Position t attends,
// causally, the blocks selected for it (its own block t/64 last), plain or
// with each historical block scaled by its continuous gate.
//
// One 256-thread workgroup per (64-query block, KV head, group of up to 4
// query heads).  The workgroup marks the union of its queries' selections in
// an LDS bitmap and walks it in ascending block order.  Each visited block's
// K and V rows (32 KiB) are staged once in LDS and shared by the 4 waves; the
// next block's loads are in flight while the current one is consumed (two
// stages).  Wave w owns queries 16w .. 16w+15 of the block and the group's
// heads:
//   S^T (64 keys x 16 queries) = K . Q^T per head with
//     v_mfma_f32_16x16x32_bf16, K read from LDS as the A operand (272-byte
//     row pitch: conflict-free 16-byte reads);
//   the lane of a query that did not select the block masks its column to
//     -inf; the query's own block is masked causally (key <= query);
//   online softmax in the log2 domain; O^T += V^T . P^T, V^T read with
//     ds_read_b64_tr_b16 from a 288-byte-pitch tile.
// A wave none of whose 16 queries selected the block skips its arithmetic.
// The work is a dense contraction per visited block: 4 heads x (64 QK + 64
// PV) MFMAs per wave.
#include <limits.h>

#include "sas_device.h"
#include "sas_kernels.h"

namespace sas {
namespace {

constexpr int kThreads = 256;
constexpr int kChunks = 64 * (kHeadDim * 2 / 16) / kThreads;  // 16-byte pieces of K (and V) per thread: 4
constexpr int kKPitch = 272;
constexpr int kVPitchP = 288;
constexpr int kKTile = kBlock * kKPitch;
constexpr int kStage = kKTile + kBlock * kVPitchP;  // 35 KiB

__device__ __forceinline__ bf16x8 as_bf16(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t pack_rne(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, b16x2));
}

}  // namespace

template <bool kGated>
__global__ __launch_bounds__(kThreads, 1) void prefill_attend_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[2][kStage];
  __shared__ uint32_t bm[SAS_MAX_BLOCKS_DEV / 32];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4, j = lane & 15;
  const int G = p.group;
  // blockIdx -> (query block, KV head, head group): heaviest query blocks
  // first, consecutive workgroups on different KV heads
  const int hg = blockIdx.x % p.head_groups;
  const int rest = blockIdx.x / p.head_groups;
  const int kvh = rest % p.n_kv_heads;
  const int qb = p.n_qblocks - 1 - rest / p.n_kv_heads;
  const int nh = min(4, G - 4 * hg);  // heads of this workgroup (>= 1)
  const int T = p.seq_len;
  const int t0 = qb * kBlock;
  const int nq = min(kBlock, T - t0);
  const int qi = 16 * wave + j;  // this lane's query within the block
  const bool qvalid = qi < nq;
  const int tq = t0 + qi;

  // ---- union of the block's selections (blocks 0 .. qb)
  const int nwords = (qb + 32) >> 5;
  for (int i = tid; i < nwords; i += kThreads) bm[i] = 0;
  __syncthreads();
  for (int e = tid; e < nq * p.max_sel; e += kThreads) {
    const int q = e / p.max_sel, slot = e - q * p.max_sel;
    const int64_t u = (int64_t)(t0 + q) * p.n_kv_heads + kvh;
    if (slot < p.cnt[u]) {
      const int c = p.sel[u * p.max_sel + slot];
      if ((unsigned)c <= (unsigned)qb) atomicOr(&bm[c >> 5], 1u << (c & 31));
    }
  }
  __syncthreads();

  // ---- this lane's walk through its query's ascending selection
  const int64_t uq = (int64_t)(qvalid ? tq : t0) * p.n_kv_heads + kvh;
  const int32_t *selq = p.sel + uq * p.max_sel;
  const float *gq = kGated ? p.gates + uq * p.max_sel : nullptr;
  const int cq = qvalid ? p.cnt[uq] : 0;
  int ptr = 0;
  int nxt_c = cq > 0 ? selq[0] : INT_MAX;
  float nxt_g = (kGated && cq > 0) ? gq[0] : 1.f;

  // B operand of S^T = K Q^T: lane l holds q[query qi][head][32ks + 8(l/16) .. +7]
  bf16x8 qB[4][4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const bool ok = qvalid && ct < nh;
    const uint16_t *qrow = p.q + ((int64_t)(ok ? tq : 0) * p.n_q_heads + kvh * G + 4 * hg + (ok ? ct : 0)) * kHeadDim + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qB[ct][ks] = as_bf16(ok ? ld16(qrow + 32 * ks) : u32x4{0, 0, 0, 0});
  }
  f32x4 o[4][8];
  float m[4], ls[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[ct] = -__builtin_inff();
    ls[ct] = 0.f;
  }

  const char *kbase = reinterpret_cast<const char *>(p.k_pool) + (int64_t)kvh * p.head_stride * 2;
  const char *vbase = reinterpret_cast<const char *>(p.v_pool) + (int64_t)kvh * p.head_stride * 2;
  const int64_t tok_bytes = p.tok_stride * 2, page_bytes = p.page_stride * 2;
  u32x4 kr[kChunks], vr[kChunks];
  auto issue = [&](int c) {  // the block's K and V rows into registers (chunk i: row i/16, bytes 16(i%16))
    const int64_t off = (int64_t)p.block_table[c] * page_bytes;
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      const int i = tid + kThreads * k;
      const int64_t a = off + (i >> 4) * tok_bytes + 16 * (i & 15);
      kr[k] = ld16(kbase + a);
      vr[k] = ld16(vbase + a);
    }
  };
  auto park = [&](int c, uint8_t *st) {  // registers -> LDS stage; V rows past the sequence end are zeroed
    const int nvalid = min(kBlock, T - c * kBlock);
#pragma unroll
    for (int k = 0; k < kChunks; ++k) {
      const int i = tid + kThreads * k;
      const int row = i >> 4, col = i & 15;
      *reinterpret_cast<u32x4 *>(st + row * kKPitch + 16 * col) = kr[k];
      *reinterpret_cast<u32x4 *>(st + kKTile + row * kVPitchP + 16 * col) =
          row < nvalid ? vr[k] : u32x4{0, 0, 0, 0};
    }
  };
  // uniform cursor over the bitmap
  int wi = 0;
  uint32_t bits = __builtin_amdgcn_readfirstlane(bm[0]);
  auto next_block = [&]() -> int {
    while (bits == 0) {
      if (++wi >= nwords) return -1;
      bits = __builtin_amdgcn_readfirstlane(bm[wi]);
    }
    const int c = (wi << 5) + __builtin_ctz(bits);
    bits &= bits - 1;
    return c;
  };

  const int tr_e = (lane & 15) >> 2, tr_q = lane & 3;
  int c = next_block();  // never -1: every query selects its own block
  int buf = 0;
  issue(c);
  park(c, stage[0]);
  __syncthreads();
  while (c >= 0) {
    const int cn = next_block();
    if (cn >= 0) issue(cn);
    // ---- attend block c from stage[buf]
    const bool s_l = nxt_c == c;
    const float g_l = s_l ? nxt_g : 0.f;
    if (s_l) {
      ++ptr;
      nxt_c = ptr < cq ? selq[ptr] : INT_MAX;
      if (kGated) nxt_g = ptr < cq ? gq[ptr] : 1.f;
    }
    if (__builtin_amdgcn_ballot_w64(s_l) != 0) {
      const uint8_t *kt = stage[buf];
      const uint8_t *vt = stage[buf] + kKTile;
      f32x4 sacc[4][4];  // [head][key tile]
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        u32x4 ka[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          ka[ks] = *reinterpret_cast<const u32x4 *>(kt + (16 * t + j) * kKPitch + 64 * ks + 16 * g);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          sacc[ct][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            sacc[ct][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16(ka[ks]), qB[ct][ks], sacc[ct][t], 0, 0, 0);
        }
      }
      const bool causal = c == qb;
      u32x4 pB[4][2];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        float z[4][4];
        float mx = -__builtin_inff();
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tau = 16 * t + 4 * g + r;
            const bool keep = s_l && (!causal || tau <= qi);
            z[t][r] = keep ? sacc[ct][t][r] * p.scale_log2 : -__builtin_inff();
            mx = fmaxf(mx, z[t][r]);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m[ct], mx);
        const bool live = m_new != -__builtin_inff();
        const float alpha = live ? exp2f(m[ct] - m_new) : 1.0f;
        float psum = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          float pv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int t = 2 * s2 + (e >> 2), r = e & 3;
            const float pe = live ? exp2f(z[t][r] - m_new) : 0.f;
            psum += pe;
            pv[e] = kGated ? pe * g_l : pe;
          }
          pB[ct][s2] = u32x4{pack_rne(pv[0], pv[1]), pack_rne(pv[2], pv[3]), pack_rne(pv[4], pv[5]),
                             pack_rne(pv[6], pv[7])};
        }
        ls[ct] = ls[ct] * alpha + psum;
        m[ct] = m_new;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[ct][dt] *= alpha;
      }
      // tr-read lane roles: within the 16-lane group g, lane 4e+q4 addresses
      // row 4g+e (+16 for the upper half of the k-step, +32 per k-step),
      // columns 16dt + 4q4 .. +3
      const uint8_t *vrd = vt + (4 * g + tr_e) * kVPitchP + 8 * tr_q;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4 *)(vrd + 32 * s2 * kVPitchP + 32 * dt));
          i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4 *)(vrd + (32 * s2 + 16) * kVPitchP + 32 * dt));
          u32x2 lo2 = __builtin_bit_cast(u32x2, a0), hi2 = __builtin_bit_cast(u32x2, a1);
          const bf16x8 a = as_bf16(u32x4{lo2.x, lo2.y, hi2.x, hi2.y});
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            o[ct][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16(pB[ct][s2]), o[ct][dt], 0, 0, 0);
        }
      }
    }
    if (cn >= 0) park(cn, stage[buf ^ 1]);
    lds_barrier();
    buf ^= 1;
    c = cn;
  }

  // ---- normalise and store: lane holds dims 16dt + 4(l/16) .. +3 of its query
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    float l = ls[ct];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (qvalid && ct < nh) {
      const float inv = 1.0f / l;
      uint16_t *dst = p.out + ((int64_t)tq * p.n_q_heads + kvh * G + 4 * hg + ct) * kHeadDim + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const f32x4 v = o[ct][dt] * inv;
        *reinterpret_cast<u32x2 *>(dst + 16 * dt) = u32x2{pack_rne(v[0], v[1]), pack_rne(v[2], v[3])};
      }
    }
  }
}

hipError_t launch_prefill_attend(const PrefillParams &p, hipStream_t st) {
  const dim3 grid((unsigned)(p.n_qblocks * p.n_kv_heads * p.head_groups));
  if (p.gates)
    hipLaunchKernelGGL((prefill_attend_kernel<true>), grid, dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL((prefill_attend_kernel<false>), grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace sas
