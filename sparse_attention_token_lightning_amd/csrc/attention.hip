// Sparse-attention consumer: each request's heads attend the k cache rows its
// indexer selected.
//
// Sources: "IndexCache: Cross-Layer Index Reuse for Sparse Attention", Symbol
// Map (the selected set holds the k positions sent to core sparse attention);
// "Multi-layer Indexer: Overlapping Selection and Attention in DeepSeek Sparse
// Attention", The abstract and The Brief (attention consumes the selection;
// the indexer can run on a second stream beside it).  The attention's form is
// not on the pages; it is read as the latent decode attention of the pages'
// model: one cached row of Dk = 576 values per token, shared by all heads, as
// the key, and its first Dv = 512 values as the value:
//     o[b][h] = sum_j p_j kv[r_j][0:512] / sum_j p_j,  p_j = exp(s_j - max s),
//     s_j = scale * (q[b][h] . kv[r_j]),  r_j = kv_off[b] + idx[b][j] (idx >= 0).
//
// Both products run on bf16 MFMA (v_mfma_f32_16x16x32_bf16).  A workgroup
// takes one request, 64 heads (16 per wave) and a range of 32-token tiles; the
// scores are computed transposed, S^T = K Q^T (tokens x heads), with the
// query in registers.  The tokens of a tile are assigned to the rows of the
// two 16-token score products so that each lane ends up holding the scores of
// 8 consecutive tokens for one head, exactly the P operand of O = P V: no lane
// exchange between the two products.  V is transposed in registers (8 tokens
// x 8 values per thread) into a tokens-along-K LDS layout for the B operand.
// The softmax is online (running max and sum per head); splits of the token
// range write unnormalised partial outputs that a second kernel combines in a
// fixed order.
#include "li_device.h"
#include "li_internal.h"

namespace li {
namespace {

constexpr int kAtDk = 576;
constexpr int kAtDv = 512;
constexpr int kAtKb = kAtDk / 32;  // 18 K blocks of the score product
constexpr int kAtDt = kAtDv / 16;  // 32 value tiles of the output product
constexpr int kAtTok = 32;         // tokens per tile
constexpr int kAtThreads = 256;    // 4 waves x 16 heads

// LDS slot address with one 16-byte pad per 16 slots: fragment reads (64
// consecutive slots) stay contiguous per 8 lanes, and the producers' stride-16
// slot writes spread over the banks.
__device__ __forceinline__ int at_pad(int slot) { return slot + (slot >> 4); }

// Transpose of an 8 x 8 block of 16-bit values: in[j] holds row j (8 values
// in 4 words); out[e] gets column e (8 values, row j in position j).
__device__ __forceinline__ void transpose8x8(const i32x4 (&in)[8], i32x4 (&out)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int w = e >> 1;
    // v_perm byte selectors: bytes 0-3 from the second operand, 4-7 from the first
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      out[e][p] = (int)__builtin_amdgcn_perm((uint32_t)in[2 * p + 1][w], (uint32_t)in[2 * p][w], sel);
  }
}

__global__ __launch_bounds__(kAtThreads, 1) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* kv, const int32_t* __restrict__ idx,
    const int64_t* __restrict__ kv_off, int32_t H, int32_t K, float scale, int32_t tiles_per_split,
    float* __restrict__ o_part, float* __restrict__ ml_part) {
  // K operand of the score product: slot (tt * 18 + kb) * 64 + lane holds the 8
  // key values kb*32 + 8*(lane >> 4) .. +7 of the token feeding row lane & 15 of
  // 16-token product tt.  V operand: slot dt * 64 + lane holds tokens
  // 8*(lane >> 4) .. +7 of value dt*16 + (lane & 15).
  constexpr int kKSlots = 2 * kAtKb * 64, kVSlots = kAtDt * 64;
  __shared__ i32x4 lk[kKSlots + kKSlots / 16];
  __shared__ i32x4 lv[kVSlots + kVSlots / 16];
  __shared__ int vflag[kAtTok];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int hgroups = H / 64;
  const int b = blockIdx.x / hgroups, hg = blockIdx.x % hgroups;
  const int g = lane >> 4, hl = lane & 15;
  const int h = hg * 64 + wave * 16 + hl;  // this lane's head in the score layout
  const int ntiles = (K + kAtTok - 1) / kAtTok;
  const int t0 = blockIdx.y * tiles_per_split;
  const int t1 = min(t0 + tiles_per_split, ntiles);
  const int64_t base = kv_off[b];
  const int32_t* irow = idx + (int64_t)b * K;

  // the query, as the B operand of S^T = K Q^T: column = head, K = key values
  bf16x8 qf[kAtKb];
  {
    const uint16_t* qp = q + ((int64_t)b * H + h) * kAtDk + 8 * g;
#pragma unroll
    for (int kb = 0; kb < kAtKb; ++kb) qf[kb] = __builtin_bit_cast(bf16x8, ld16(qp + kb * 32));
  }

  // Gather: thread (tg = wave, c = lane) loads value chunk c (8 values) of the
  // tile's tokens 8*tg .. +7; thread tid also loads chunk 64 + (tid & 7) (the
  // last 64 key values) of token tid >> 3.
  const int tg = wave, c = lane;
  const int xt = tid >> 3, xc = 64 + (tid & 7);
  i32x4 gv[8], gx;
  int xvalid = 0;
  auto row_of = [&](int slot, bool& valid) -> int64_t {
    const int32_t t = slot < K ? irow[slot] : -1;
    valid = t >= 0;
    return valid ? base + t : 0;  // an invalid slot reads row 0: loaded, then masked
  };
  auto gather = [&](int tile) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bool v;
      const int64_t r = row_of(tile * kAtTok + 8 * tg + j, v);
      gv[j] = ld16(kv + r * kAtDk + 8 * c);
    }
    bool v;
    const int64_t r = row_of(tile * kAtTok + xt, v);
    gx = ld16(kv + r * kAtDk + 8 * xc);
    xvalid = v;
  };
  // token tau of the tile feeds row 4*(tau >> 3) + (tau & 3) of product (tau >> 2) & 1
  auto kslot = [&](int tau, int chunk) {
    const int tt = (tau >> 2) & 1, r = 4 * (tau >> 3) + (tau & 3);
    return at_pad((tt * kAtKb + (chunk >> 2)) * 64 + (chunk & 3) * 16 + r);
  };
  auto stage = [&]() {
#pragma unroll
    for (int j = 0; j < 8; ++j) lk[kslot(8 * tg + j, c)] = gv[j];
    lk[kslot(xt, xc)] = gx;
    if ((tid & 7) == 0) vflag[xt] = xvalid;
    i32x4 tr[8];
    transpose8x8(gv, tr);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * c + e;  // value index
      lv[at_pad((d >> 4) * 64 + tg * 16 + (d & 15))] = tr[e];
    }
  };

  f32x4 oacc[kAtDt];
#pragma unroll
  for (int dt = 0; dt < kAtDt; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  if (t0 < t1) gather(t0);
  for (int tile = t0; tile < t1; ++tile) {
    __syncthreads();  // the previous tile's LDS reads are done
    stage();
    __syncthreads();
    if (tile + 1 < t1) gather(tile + 1);

    // S^T for this wave's 16 heads: two 16-token products
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kb = 0; kb < kAtKb; ++kb) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, lk[at_pad((tt * kAtKb + kb) * 64 + lane)]);
        sacc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[kb], sacc[tt], 0, 0, 0);
      }
    }
    // lane (g, hl): sacc[tt][i] is token 8g + 4tt + i of the tile, head hl
    float s[8];
    float mloc = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool ok = vflag[8 * g + j] != 0;
      s[j] = ok ? sacc[j >> 2][j & 3] * scale : -INFINITY;
      mloc = fmaxf(mloc, s[j]);
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float m_new = fmaxf(m_run, mloc);
    const bool any = m_new != -INFINITY;
    const float alpha = any ? __expf(m_run - m_new) : 1.f;
    m_run = m_new;
    float psum = 0.f;
    bf16x8 pa;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = any ? __expf(s[j] - m_new) : 0.f;
      const __bf16 pb = (__bf16)p;
      pa[j] = pb;
      psum += (float)pb;  // the sum uses the rounded weights the product uses
    }
    l_run = l_run * alpha + psum;
    // rescale the output rows (heads 4g + i in the output layout) by their alpha
    if (__ballot(alpha != 1.f) != 0) {  // wave-uniform: skip when no head's max moved
      float a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
      for (int dt = 0; dt < kAtDt; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[dt][i] *= a[i];
    }
    // O += P V
#pragma unroll
    for (int dt = 0; dt < kAtDt; ++dt) {
      const bf16x8 vf = __builtin_bit_cast(bf16x8, lv[at_pad(dt * 64 + lane)]);
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vf, oacc[dt], 0, 0, 0);
    }
  }

  // partial results of this split: unnormalised o, running max and sum
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  const int64_t prow = ((int64_t)blockIdx.y * (gridDim.x / hgroups) + b) * H + hg * 64 + wave * 16;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float* op = o_part + (prow + 4 * g + i) * kAtDv + hl;
#pragma unroll
    for (int dt = 0; dt < kAtDt; ++dt) op[dt * 16] = oacc[dt][i];
  }
  if (g == 0) {
    ml_part[(prow + hl) * 2] = m_run;
    ml_part[(prow + hl) * 2 + 1] = l_run;
  }
}

// o[b][h] = sum_s e_s o_s / sum_s e_s l_s with e_s = exp(m_s - max m), splits
// in order; 0 when no split saw a selected token.  One workgroup per (b, h).
__global__ __launch_bounds__(128) void sparse_attn_combine_kernel(const float* __restrict__ o_part,
                                                                  const float* __restrict__ ml_part, int32_t S,
                                                                  int64_t rows, float* __restrict__ out) {
  const int64_t row = blockIdx.x;
  float m = -INFINITY;
  for (int s = 0; s < S; ++s) m = fmaxf(m, ml_part[(s * rows + row) * 2]);
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  if (m != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float ms = ml_part[(s * rows + row) * 2];
      const float e = ms == -INFINITY ? 0.f : __expf(ms - m);
      l += e * ml_part[(s * rows + row) * 2 + 1];
      const f32x4 v = *reinterpret_cast<const f32x4*>(o_part + (s * rows + row) * kAtDv + 4 * threadIdx.x);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] += e * v[k];
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  f32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) r[k] = acc[k] * inv;
  *reinterpret_cast<f32x4*>(out + row * kAtDv + 4 * threadIdx.x) = r;
}

}  // namespace

int32_t attention_splits(int32_t B, int32_t H, int32_t K) {
  const int32_t units = B * (H / 64);
  const int32_t ntiles = (K + kAtTok - 1) / kAtTok;
  int32_t s = (256 + units - 1) / units;
  if (s > ntiles) s = ntiles;
  if (s < 1) s = 1;
  const int32_t per = (ntiles + s - 1) / s;
  return (ntiles + per - 1) / per;
}

hipError_t launch_sparse_attention(const uint16_t* q, const uint16_t* kv, const int32_t* idx, const int64_t* kv_off,
                                   int32_t B, int32_t H, int32_t K, float scale, float* o_part, float* ml_part,
                                   float* out, hipStream_t stream) {
  const int32_t S = attention_splits(B, H, K);
  const int32_t ntiles = (K + kAtTok - 1) / kAtTok;
  const int32_t per = (ntiles + S - 1) / S;
  const dim3 grid((unsigned)(B * (H / 64)), (unsigned)S);
  hipError_t e = launch_kernel(sparse_attn_kernel, grid, dim3(kAtThreads), 0, stream, q, kv, idx, kv_off, H, K, scale,
                               per, o_part, ml_part);
  if (e != hipSuccess) return e;
  return launch_kernel(sparse_attn_combine_kernel, dim3((unsigned)(B * H)), dim3(kAtDv / 4), 0, stream,
                       (const float*)o_part, (const float*)ml_part, S, (int64_t)B * H, out);
}

}  // namespace li
