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
// takes one request, 64 heads and a range of 32-token tiles; each of its 8
// waves has 16 heads and half of the 512 values (the two waves of a head tile
// compute the same scores), so two waves share each SIMD; the
// scores are computed transposed, S^T = K Q^T (tokens x heads), with the
// query in registers.  The tokens of a tile are assigned to the rows of the
// two 16-token score products so that each lane ends up holding the scores of
// 8 consecutive tokens for one head, exactly the P operand of O = P V: no lane
// exchange between the two products.  V is transposed in registers (4 tokens
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
constexpr int kAtThreads = 512;    // 8 waves: 4 head tiles x 2 halves of the values
constexpr int kAtMaxTiles = 64;    // tiles per split (its selection is staged in LDS)
constexpr float kAtSlack = 8.f;    // the reference max moves only when a max exceeds it by more

// LDS slot address with one 16-byte pad per 16 slots: fragment reads (64
// consecutive slots) stay contiguous per 8 lanes, and the producers' stride-16
// slot writes spread over the banks.
__device__ __forceinline__ int at_pad(int slot) { return slot + (slot >> 4); }

// V tile address: the padded slot with its place in the 16-slot block XOR-ed
// by bits 6..9 of the slot.  Fragment reads stay conflict-free (a permutation
// within each block), and the transposed 8-byte writes, which otherwise land
// 16 lanes on 4 bank groups, hit each bank at most twice per 32 lanes.
__device__ __forceinline__ int at_swz(int slot) { return 17 * (slot >> 4) + ((slot & 15) ^ ((slot >> 6) & 15)); }

// Transpose of a 4 x 8 block of 16-bit values: in[j] holds row j (8 values in
// 4 words); out[e] gets column e (4 values, row j in position j).
__device__ __forceinline__ void transpose4x8(const i32x4 (&in)[4], i32x2 (&out)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int w = e >> 1;
    // v_perm byte selectors: bytes 0-3 from the second operand, 4-7 from the first
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
    out[e][0] = (int)__builtin_amdgcn_perm((uint32_t)in[1][w], (uint32_t)in[0][w], sel);
    out[e][1] = (int)__builtin_amdgcn_perm((uint32_t)in[3][w], (uint32_t)in[2][w], sel);
  }
}

__global__ __launch_bounds__(kAtThreads, 1) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* kv, const int32_t* __restrict__ idx,
    const int64_t* __restrict__ kv_off, int32_t B, int32_t H, int32_t K, float scale, int32_t tiles_per_split,
    float* __restrict__ o_part, float* __restrict__ ml_part) {
  // K operand of the score product: slot (tt * 18 + kb) * 64 + lane holds the 8
  // key values kb*32 + 8*(lane >> 4) .. +7 of the token feeding row lane & 15 of
  // 16-token product tt.  V operand: slot dt * 64 + lane holds tokens
  // 8*(lane >> 4) .. +7 of value dt*16 + (lane & 15).
  constexpr int kKSlots = 2 * kAtKb * 64, kVSlots = kAtDt * 64;
  __shared__ i32x4 lk[kKSlots + kKSlots / 16];
  __shared__ i32x4 lv[kVSlots + kVSlots / 16];
  __shared__ int32_t lidx[kAtMaxTiles * kAtTok];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int ht = wave & 3, dh = wave >> 2;  // head tile (16 heads), half of the values (16 value tiles)
  const int hgroups = H / 64;
  const int b = blockIdx.x / hgroups, hg = blockIdx.x % hgroups;
  const int g = lane >> 4, hl = lane & 15;
  const int h = hg * 64 + ht * 16 + hl;  // this lane's head in the score layout
  const int ntiles = (K + kAtTok - 1) / kAtTok;
  const int t0 = blockIdx.y * tiles_per_split;
  const int t1 = min(t0 + tiles_per_split, ntiles);
  const int64_t base = kv_off[b];
  const int32_t* irow = idx + (int64_t)b * K;

  // The split's selection, once, into LDS (at most kAtMaxTiles tiles): the row
  // of every gather is then one LDS read away, not a dependent global load.
  for (int i = tid; i < (t1 - t0) * kAtTok; i += kAtThreads) {
    const int slot = t0 * kAtTok + i;
    lidx[i] = slot < K ? irow[slot] : -1;
  }

  // the query, as the B operand of S^T = K Q^T: column = head, K = key values
  bf16x8 qf[kAtKb];
  {
    const uint16_t* qp = q + ((int64_t)b * H + h) * kAtDk + 8 * g;
#pragma unroll
    for (int kb = 0; kb < kAtKb; ++kb) qf[kb] = __builtin_bit_cast(bf16x8, ld16(qp + kb * 32));
  }
  __syncthreads();

  // Gather: thread (tq = wave, c = lane) loads value chunk c (8 values) of the
  // tile's tokens 4*tq .. +3; threads tid < 256 also load chunk 64 + (tid & 7)
  // (the last 64 key values) of token tid >> 3.
  const int tq = wave, c = lane;
  const bool xthr = tid < 256;
  const int xt = (tid & 255) >> 3, xc = 64 + (tid & 7);
  i32x4 gv[4], gx;
  auto row_at = [&](int tile, int tau) -> int64_t {
    const int32_t t = lidx[(tile - t0) * kAtTok + tau];
    return t >= 0 ? base + t : 0;  // an unselected slot reads row 0: loaded, then masked
  };
  auto gather = [&](int tile) {
    int64_t r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = row_at(tile, 4 * tq + j);
#pragma unroll
    for (int j = 0; j < 4; ++j) gv[j] = ld16(kv + r[j] * kAtDk + 8 * c);
    if (xthr) gx = ld16(kv + row_at(tile, xt) * kAtDk + 8 * xc);
  };
  // token tau of the tile feeds row 4*(tau >> 3) + (tau & 3) of product (tau >> 2) & 1
  auto kslot = [&](int tau, int chunk) {
    const int tt = (tau >> 2) & 1, r = 4 * (tau >> 3) + (tau & 3);
    return at_pad((tt * kAtKb + (chunk >> 2)) * 64 + (chunk & 3) * 16 + r);
  };
  auto stage = [&]() {
#pragma unroll
    for (int j = 0; j < 4; ++j) lk[kslot(4 * tq + j, c)] = gv[j];
    if (xthr) lk[kslot(xt, xc)] = gx;
    i32x2 tr[8];
    transpose4x8(gv, tr);
    i32x2* lv2 = reinterpret_cast<i32x2*>(lv);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * c + e;  // value index; tokens 4*tq .. +3 are half (tq & 1) of group tq >> 1
      lv2[2 * at_swz((d >> 4) * 64 + (tq >> 1) * 16 + (d & 15)) + (tq & 1)] = tr[e];
    }
  };

  constexpr int kHalf = kAtDt / 2;
  f32x4 oacc[kHalf];
#pragma unroll
  for (int dt = 0; dt < kHalf; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY, l_run = 0.f;

  auto compute = [&](int tile) {
    // S^T for this wave's 16 heads: two 16-token products, each summed over the
    // 18 K blocks in two independent chains
    f32x4 sacc[2][2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) sacc[tt][ch] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < kAtKb; ++kb) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, lk[at_pad((tt * kAtKb + kb) * 64 + lane)]);
        sacc[tt][kb & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[kb], sacc[tt][kb & 1], 0, 0, 0);
      }
    }
    // lane (g, hl): token 8g + 4tt + i of the tile, head hl
    float s[8];
    float mloc = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tt = j >> 2, i = j & 3;
      const float v = sacc[tt][0][i] + sacc[tt][1][i];
      const bool ok = lidx[(tile - t0) * kAtTok + 8 * g + j] >= 0;
      s[j] = ok ? v * scale : -INFINITY;
      mloc = fmaxf(mloc, s[j]);
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    // Lazy reference: the weights are exp(s - m_ref); m_ref moves (and the
    // output is rescaled) only when a score exceeds it by more than kAtSlack,
    // so weights stay below e^kAtSlack and the softmax is unchanged.
    const bool move = mloc > m_ref + kAtSlack || (m_ref == -INFINITY && mloc != -INFINITY);
    const float m_new = move ? mloc : m_ref;
    const float alpha = move ? __expf(m_ref - m_new) : 1.f;  // 0 when m_ref was -inf
    m_ref = m_new;
    const bool any = m_new != -INFINITY;
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
    if (__ballot(move) != 0) {  // wave-uniform; rows of the output layout are heads 4g + i
      float a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
      for (int dt = 0; dt < kHalf; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[dt][i] *= a[i];
    }
    // O += P V over this wave's half of the values
#pragma unroll
    for (int dt = 0; dt < kHalf; ++dt) {
      const bf16x8 vf = __builtin_bit_cast(bf16x8, lv[at_swz((dh * kHalf + dt) * 64 + lane)]);
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vf, oacc[dt], 0, 0, 0);
    }
  };

  if (t0 < t1) gather(t0);
  for (int tile = t0; tile < t1; ++tile) {
    __syncthreads();  // the previous tile's LDS reads are done
    stage();
    __syncthreads();
    if (tile + 1 < t1) gather(tile + 1);
    compute(tile);
  }

  // partial results of this split: unnormalised o, reference max and sum
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  const int64_t prow = ((int64_t)blockIdx.y * B + b) * H + hg * 64 + ht * 16;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float* op = o_part + (prow + 4 * g + i) * kAtDv + dh * (kAtDv / 2) + hl;
#pragma unroll
    for (int dt = 0; dt < kHalf; ++dt) op[dt * 16] = oacc[dt][i];
  }
  if (dh == 0 && g == 0) {
    ml_part[(prow + hl) * 2] = m_ref;
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
  if (s < (ntiles + kAtMaxTiles - 1) / kAtMaxTiles) s = (ntiles + kAtMaxTiles - 1) / kAtMaxTiles;
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
  hipError_t e = launch_kernel(sparse_attn_kernel, grid, dim3(kAtThreads), 0, stream, q, kv, idx, kv_off, B, H, K,
                               scale, per, o_part, ml_part);
  if (e != hipSuccess) return e;
  return launch_kernel(sparse_attn_combine_kernel, dim3((unsigned)(B * H)), dim3(kAtDv / 4), 0, stream,
                       (const float*)o_part, (const float*)ml_part, S, (int64_t)B * H, out);
}

}  // namespace li
