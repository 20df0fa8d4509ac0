// Key-block pooling -> gate keys.
//
// SAS pools each 64-token key block by max, min and average and maps the
// pooled statistics to a 128-wide gate key with Q/K normalisation and gate
// RoPE ("Tencent released Simple-Attention-Sparsification ...", aigc.news,
// the setup paragraph; "Specifications and Configuration Table" of the
// localmodelwatch model page: KV block size 64, gate hidden size 128, key
// block pooling max + min + average, Q/K normalization, gate RoPE).
//
// One workgroup (256 threads) per (16 listed blocks, KV head):
//   1. thread (block t/16, dims 8(t%16) .. +7) scans its block's 64 key rows
//      with 16-byte loads: max, min and an fp32 sum in row order ->
//      pooled[b][384] = [max | min | mean] in LDS;
//   2. U^T = w_k[h] . P^T (128 x 384 times 384 x 16 blocks) on MFMA: the max
//      and min inputs are bf16 values, the means are split into bf16 high and
//      low parts (about 16 significant bits); w_k is read once per 16 blocks;
//   3. per block: RMSNorm (eps 1e-6) * w_knorm, rotate-half RoPE at position
//      64*c (angles formed and reduced in fp64), round to bf16, store.
// Bytes per (block, KV head): 16 KiB of keys read, 256 B of gate key written
// (w_k, 96 KiB per KV head, is read from L2 once per 16 blocks).
//
// The same pooling also runs inside the decode step's cache write
// (append_kernel): the step that writes a block's last row pools the block
// there, instead of a second launch re-reading that row.  It runs the same
// arithmetic on a batch of one block, so its gate keys are bit-identical.
#include "sas_device.h"
#include "sas_kernels.h"

namespace sas {
namespace {

constexpr int kPoolBatch = 16;                // blocks per workgroup
constexpr int kPoolAhead = 16;                // key rows each thread keeps in flight
constexpr int kPooledPitch = 3 * kHeadDim + 4;  // LDS row of pooled statistics (floats), staggered banks
constexpr int kUPitch = kGateDim + 4;

__device__ __forceinline__ bf16x8 as_b8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

}  // namespace

// Gate keys of nb <= 16 key blocks of one KV head.  Every thread of a
// 256-thread workgroup calls it (it holds barriers).  src[b]: element offset
// of block b's row 0 of this head in k_pool; blk[b]: its block index (RoPE
// position 64 blk[b]); dst[b]: element offset of its 128 gate-key values in
// gate_keys; all three in LDS, written by the caller before a barrier.
// (Offsets rather than pointers: addresses formed from the kernel's buffer
// arguments compile to global loads, whose waits count only the loads
// before them; pointers read back from LDS would compile to flat loads,
// which the compiler drains completely before any use.)  last_row: when non-null, block 0's row 63 is read from there
// instead of from the pool (the append kernel passes the row it is writing).
__device__ __forceinline__ void pool_batch(int nb, const uint16_t *k_pool, const int64_t *src, const int *blk,
                                           uint16_t *gate_keys, const int64_t *dst,
                           int64_t tok_stride, const uint16_t *last_row, const uint16_t *w_kh,
                           const float *w_knorm, double theta) {
  __shared__ __attribute__((aligned(16))) float pooled[kPoolBatch][kPooledPitch];
  __shared__ float uk[kPoolBatch][kUPitch];
  __shared__ double invf[kGateDim / 2];
  __shared__ float wkn[kGateDim];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int b = t >> 4, o = t & 15;

  if (t < kGateDim / 2) invf[t] = pow(theta, -(double)t / 64.0);
  if (t < kGateDim) wkn[t] = w_knorm[t];

  // ---- 1. pooled statistics
  if (b < nb) {
    const uint16_t *kb = k_pool + src[b] + 8 * o;
    float mx[8], mn[8], sum[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      mx[e] = -__builtin_inff();
      mn[e] = __builtin_inff();
      sum[e] = 0.f;
    }
    // a rolling window of kPoolAhead rows in flight: row r + kPoolAhead is
    // issued as soon as row r is consumed (rows summed in order)
    auto row = [&](int r) {
      return (last_row && b == 0 && r == kBlock - 1) ? ld16(last_row + 8 * o) : ld16(kb + (int64_t)r * tok_stride);
    };
    u32x4 win[kPoolAhead];
#pragma unroll
    for (int r = 0; r < kPoolAhead; ++r) win[r] = row(r);
#pragma unroll
    for (int r = 0; r < kBlock; ++r) {
      const u32x4 w = win[r % kPoolAhead];
      if (r + kPoolAhead < kBlock) win[r % kPoolAhead] = row(r + kPoolAhead);
      const float x[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                          bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        mx[e] = fmaxf(mx[e], x[e]);
        mn[e] = fminf(mn[e], x[e]);
        sum[e] += x[e];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pooled[b][8 * o + e] = mx[e];
      pooled[b][kHeadDim + 8 * o + e] = mn[e];
      pooled[b][2 * kHeadDim + 8 * o + e] = sum[e] * (1.0f / kBlock);
    }
  }
  // w_k A operands of this wave's 32 output rows (row 32w + 16mt + l%16,
  // inputs 32ks + 8(l/16) .. +7), loaded after the key scan so that the two
  // never hold registers together (several workgroups then share a CU)
  u32x4 wk[2][12];
  {
    const uint16_t *w = w_kh + (int64_t)(32 * wave + (lane & 15)) * 3 * kHeadDim + 8 * (lane >> 4);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int ks = 0; ks < 12; ++ks) wk[mt][ks] = ld16(w + (int64_t)16 * mt * 3 * kHeadDim + 32 * ks);
  }
  lds_barrier();

  // ---- 2. U^T = w_k P^T: lane l holds block l%16, rows 32w + 16mt + 4(l/16) + r
  // (columns of blocks past nb hold stale values and are not read)
  {
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
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(wk[mt][ks]), as_b8(h), acc[mt], 0, 0, 0);
      if (ks >= 8) {  // the means: add the low parts
        float lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) lo[e] = x[e] - ((e & 1) ? bf16_hi(h[e >> 1]) : bf16_lo(h[e >> 1]));
        const u32x4 l = {pack_bf16_rne(lo[0], lo[1]), pack_bf16_rne(lo[2], lo[3]), pack_bf16_rne(lo[4], lo[5]),
                         pack_bf16_rne(lo[6], lo[7])};
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_b8(wk[mt][ks]), as_b8(l), acc[mt], 0, 0, 0);
      }
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) uk[lane & 15][32 * wave + 16 * mt + 4 * (lane >> 4) + r] = acc[mt][r];
  }
  lds_barrier();

  // ---- 3. per block (16 lanes each, dims o + 16k): RMSNorm, w_knorm, RoPE at
  // position 64 blk; the bf16 results go back to LDS, then out as 16-byte rows
  if (b < nb) {
    float x[8], ss = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      x[k] = uk[b][o + 16 * k];
      ss += x[k] * x[k];
    }
    const float inv = 1.0f / sqrtf(row16_sum(ss) * (1.0f / kGateDim) + 1e-6f);
    const double pos = (double)blk[b] * kBlock;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int d = o + 16 * k;
      const float a = x[k] * inv * wkn[d], bb = x[k + 4] * inv * wkn[d + 64];
      float cf, sf;
      rope_cos_sin(pos, invf[d], cf, sf);
      uk[b][d] = a * cf - bb * sf;
      uk[b][d + 64] = bb * cf + a * sf;
    }
  }
  lds_barrier();
  if (b < nb) {
    const float *u = &uk[b][8 * o];
    *reinterpret_cast<u32x4 *>(gate_keys + dst[b] + 8 * o) =
        u32x4{pack_bf16x2(u[0], u[1]), pack_bf16x2(u[2], u[3]), pack_bf16x2(u[4], u[5]), pack_bf16x2(u[6], u[7])};
  }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void pool_kernel(PoolParams p) {
  __shared__ int64_t src_l[kPoolBatch], dst_l[kPoolBatch];
  __shared__ int blk_l[kPoolBatch];
  const int kvh = blockIdx.x % p.n_kv_heads;  // the KV heads of a batch run in consecutive workgroups
  const int i0 = (blockIdx.x / p.n_kv_heads) * kPoolBatch;
  const int nb = min(kPoolBatch, p.n - i0);
  if ((int)threadIdx.x < nb) {
    const int i = i0 + threadIdx.x;
    const int s = p.pool_seq[i], c = p.pool_blk[i];
    const int32_t page = p.block_table[(int64_t)s * p.max_blocks + c];
    src_l[threadIdx.x] = (int64_t)page * p.page_stride + (int64_t)kvh * p.head_stride;
    dst_l[threadIdx.x] = ((int64_t)page * p.n_kv_heads + kvh) * kGateDim;
    blk_l[threadIdx.x] = c;
  }
  lds_barrier();
  pool_batch(nb, p.k_pool, src_l, blk_l, p.gate_keys, dst_l, p.tok_stride, nullptr, p.w_k + (int64_t)kvh * kGateDim * 3 * kHeadDim,
             p.w_knorm, p.theta);
}

// One workgroup per (sequence, KV head): threads 0-15 write the new key row,
// 16-31 the value row (16 bytes each); when the row completes its block
// (L % 64 == 0) the whole workgroup pools that block, taking row 63 from
// k_new.  Bytes per (sequence, KV head): 512 B read + 512 B written, plus
// 16 KiB - 256 B of keys read and 256 B written per completed block.
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  __shared__ int64_t src_l[1], dst_l[1];
  __shared__ int blk_l[1];
  const int unit = blockIdx.x;
  const int s = unit / p.n_kv_heads;
  const int kvh = unit - s * p.n_kv_heads;
  const int t = threadIdx.x;
  const int L = p.seq_lens[s];
  const int pos = L - 1;
  const int c = pos / kBlock, r = pos - c * kBlock;
  const int32_t page = p.block_table[(int64_t)s * p.max_blocks + c];
  const int64_t base = (int64_t)page * p.page_stride + (int64_t)kvh * p.head_stride;
  const int64_t src = ((int64_t)s * p.n_kv_heads + kvh) * kHeadDim;
  if (t < 32) {
    const int lane = t & 15;
    const uint16_t *from = (t < 16 ? p.k_new : p.v_new) + src + 8 * lane;
    uint16_t *to = (t < 16 ? p.k_pool : p.v_pool) + base + (int64_t)r * p.tok_stride + 8 * lane;
    *(u32x4 *)to = ld16(from);
  }
  if (L % kBlock == 0) {
    if (t == 0) {
      src_l[0] = base;
      dst_l[0] = ((int64_t)page * p.n_kv_heads + kvh) * kGateDim;
      blk_l[0] = c;
    }
    lds_barrier();
    pool_batch(1, p.k_pool, src_l, blk_l, p.gate_keys, dst_l, p.tok_stride, p.k_new + src, p.w_k + (int64_t)kvh * kGateDim * 3 * kHeadDim,
               p.w_knorm, p.theta);
  }
}

hipError_t launch_pool(const PoolParams &p, hipStream_t st) {
  if (p.n == 0) return hipSuccess;
  const unsigned batches = (unsigned)((p.n + kPoolBatch - 1) / kPoolBatch);
  hipLaunchKernelGGL(pool_kernel, dim3(batches * (unsigned)p.n_kv_heads), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_append(const AppendParams &p, int batch, hipStream_t st) {
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)(batch * p.n_kv_heads)), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace sas
