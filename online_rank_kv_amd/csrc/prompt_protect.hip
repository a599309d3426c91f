// Exact-row sets of the prompt (iS-KV notes §3.1, Algorithm 1):
// the post-RoPE keys are cut into blocks of `block` tokens; the last
// `suffix_blocks` whole blocks and the partial tail are the local suffix.
// For every KV head and every other block, the anomaly score is the minimum
// over the block's tokens of the cosine between the token's key and the mean
// key of the block. Each head keeps its `per_head` lowest blocks (equal
// scores: lower block index first); P_K is the union of the kept blocks over
// heads plus the suffix, P_V every position within v_radius of P_K, W_V the
// last v_window positions.
//
//   anomaly_scores_kernel  one wave per (block, head): lane l holds features
//                          l, l + 64, ... of the block's keys; the mean, the
//                          norms and the dot products reduce over the wave.
//   select_kernel          one workgroup per head: a block's rank is the
//                          number of blocks before it in (score, index) order.
//   flags_kernel           one thread per position: the three set bits.
#include "iskv_internal.h"

#include <math.h>

namespace {

constexpr int PP_MAXB = 64;   // largest block
constexpr int PP_MAXDH = 256;  // largest head dimension

__device__ __forceinline__ float pp_bf(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ float pp_wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// scores[g * nb + j] for block j < nb and KV head g < Hkv (fp32 throughout).
__global__ __launch_bounds__(256) void anomaly_scores_kernel(const uint16_t* __restrict__ K, int Hkv, int dh,
                                                             int block, int nb, float* __restrict__ scores) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= nb * Hkv) return;
  const int g = item % Hkv, j = item / Hkv;
  const int D = Hkv * dh;
  constexpr int NPL = PP_MAXDH / 64;  // features per lane
  float mu[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) mu[i] = 0.f;
  const uint16_t* base = K + (size_t)j * block * D + (size_t)g * dh;
  for (int t = 0; t < block; ++t) {
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int f = lane + 64 * i;
      if (f < dh) mu[i] += pp_bf(base[(size_t)t * D + f]);
    }
  }
  float nm2 = 0.f;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    mu[i] *= 1.f / (float)block;
    nm2 = fmaf(mu[i], mu[i], nm2);
  }
  nm2 = pp_wave_sum(nm2);
  const float nm = sqrtf(nm2);
  float smin = INFINITY;
  for (int t = 0; t < block; ++t) {
    float dot = 0.f, nt2 = 0.f;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int f = lane + 64 * i;
      const float x = f < dh ? pp_bf(base[(size_t)t * D + f]) : 0.f;
      dot = fmaf(x, mu[i], dot);
      nt2 = fmaf(x, x, nt2);
    }
    dot = pp_wave_sum(dot);
    nt2 = pp_wave_sum(nt2);
    const float c = (nt2 == 0.f || nm2 == 0.f) ? 1.f : dot / (sqrtf(nt2) * nm);
    smin = fminf(smin, c);
  }
  if (lane == 0) scores[(size_t)g * nb + j] = smin;
}

// Rank order key: NaN scores sort last.
__device__ __forceinline__ float pp_key(float s) { return isnan(s) ? INFINITY : s; }

// sel[g * nb + j] = 1 when block j is among head g's per_head lowest.
__global__ __launch_bounds__(1024) void select_kernel(const float* __restrict__ scores, int nb, int per_head,
                                                      uint8_t* __restrict__ sel) {
  constexpr int TILE = 4096;
  __shared__ float ts[TILE];
  const int g = blockIdx.x;
  const float* s = scores + (size_t)g * nb;
  for (int j0 = 0; j0 < nb; j0 += blockDim.x) {
    const int j = j0 + threadIdx.x;
    const float sj = j < nb ? pp_key(s[j]) : 0.f;
    int rank = 0;
    for (int i0 = 0; i0 < nb; i0 += TILE) {
      __syncthreads();
      for (int i = threadIdx.x; i < TILE && i0 + i < nb; i += blockDim.x) ts[i] = pp_key(s[i0 + i]);
      __syncthreads();
      const int m = min(TILE, nb - i0);
      for (int i = 0; i < m; ++i) {
        const float si = ts[i];
        rank += (si < sj || (si == sj && i0 + i < j)) ? 1 : 0;
      }
    }
    if (j < nb) sel[(size_t)g * nb + j] = rank < per_head ? 1 : 0;
  }
}

// flags[p] = P_K (1) | P_V (2) | W_V (4) for prompt position p.
__global__ __launch_bounds__(256) void flags_kernel(const uint8_t* __restrict__ sel, int Hkv, int nb, int L,
                                                    int block, int v_radius, int v_window,
                                                    uint8_t* __restrict__ flags) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= L) return;
  const int s0 = nb * block;  // first suffix position
  auto in_pk = [&](int x) {
    if (x >= s0) return true;
    const int j = x / block;
    for (int g = 0; g < Hkv; ++g)
      if (sel[(size_t)g * nb + j]) return true;
    return false;
  };
  const bool pk = in_pk(p);
  bool pv = pk;
  for (int x = max(0, p - v_radius); !pv && x <= min(L - 1, p + v_radius); ++x) pv = in_pk(x);
  const bool wv = p >= L - v_window;
  flags[p] = (uint8_t)((pk ? 1 : 0) | (pv ? 2 : 0) | (wv ? 4 : 0));
}

// Split of the prompt rows by their flags (Algorithm 1): row p is
// kept exact when flags[p] & mask, else it goes to the rows the factor is
// built from; both lists stay in position order. One workgroup ranks all
// positions: thread t owns a contiguous run of them, the runs' keep counts
// are scanned over the workgroup, and dest[p] receives the row's slot
// (>= 0 in the exact list, -1 - slot in the other).
__global__ __launch_bounds__(1024) void split_scan_kernel(const uint8_t* __restrict__ flags, int L, unsigned mask,
                                                          int32_t* __restrict__ dest, int32_t* __restrict__ counts) {
  __shared__ int wsum[16];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int run = (L + 1023) / 1024;
  const int p0 = min(L, t * run), p1 = min(L, p0 + run);
  int keep = 0;
  for (int p = p0; p < p1; ++p) keep += (flags[p] & mask) ? 1 : 0;
  int incl = keep;  // inclusive scan over the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < 16; ++w) {
    before += w < wv ? wsum[w] : 0;
    total += wsum[w];
  }
  int k = before + incl - keep;  // exact rows before this run
  int rr = p0 - k;               // other rows before this run
  for (int p = p0; p < p1; ++p) dest[p] = (flags[p] & mask) ? k++ : -1 - rr++;
  if (t == 0) {
    counts[0] = total;
    counts[1] = L - total;
  }
}

// Row p moves to its slot (float4 copies) with its position pos0 + p.
__global__ __launch_bounds__(256) void split_gather_kernel(const float* __restrict__ X, int D,
                                                           const int32_t* __restrict__ dest, int pos0,
                                                           float* __restrict__ X_keep, int32_t* __restrict__ pos_keep,
                                                           float* __restrict__ X_rest, int32_t* __restrict__ pos_rest) {
  const int p = blockIdx.x;
  const int d = dest[p];
  float* out = d >= 0 ? X_keep : X_rest;
  int32_t* po = d >= 0 ? pos_keep : pos_rest;
  const int slot = d >= 0 ? d : -1 - d;
  if (!out) return;
  const float4* src = reinterpret_cast<const float4*>(X + (size_t)p * D);
  float4* dst = reinterpret_cast<float4*>(out + (size_t)slot * D);
  for (int i = threadIdx.x; i < D / 4; i += 256) dst[i] = src[i];
  if (threadIdx.x == 0 && po) po[slot] = pos0 + p;
}

inline int pp_scored_blocks(int L, int block, int suffix_blocks) {
  const int nb = L / block - suffix_blocks;
  return nb > 0 ? nb : 0;
}

}  // namespace

size_t iskv_prompt_protect_ws_bytes(int32_t L, int32_t Hkv, int32_t block, int32_t suffix_blocks) {
  if (L < 1 || Hkv < 1 || block < 1 || suffix_blocks < 0) return 0;
  const size_t nb = (size_t)pp_scored_blocks(L, block, suffix_blocks);
  return ((nb * Hkv * sizeof(float) + 255) / 256) * 256 + nb * Hkv + 256;
}

int iskv_launch_prompt_protect(const uint16_t* K_rot, int32_t L, int32_t Hkv, int32_t dh, int32_t block,
                               int32_t per_head, int32_t suffix_blocks, int32_t v_radius, int32_t v_window,
                               uint8_t* flags, float* scores_out, void* ws, size_t ws_bytes, hipStream_t s) {
  if (block > PP_MAXB || dh > PP_MAXDH) return ISKV_EINVAL;
  if (ws_bytes < iskv_prompt_protect_ws_bytes(L, Hkv, block, suffix_blocks)) return ISKV_EWORKSPACE;
  const int nb = pp_scored_blocks(L, block, suffix_blocks);
  float* sc = scores_out ? scores_out : (float*)ws;
  uint8_t* sel = (uint8_t*)ws + ((size_t)nb * Hkv * sizeof(float) + 255) / 256 * 256;
  if (nb > 0) {
    hipLaunchKernelGGL(anomaly_scores_kernel, dim3((nb * Hkv + 3) / 4), dim3(256), 0, s, K_rot, Hkv, dh, block, nb,
                       sc);
    hipLaunchKernelGGL(select_kernel, dim3(Hkv), dim3(1024), 0, s, sc, nb, per_head, sel);
  }
  hipLaunchKernelGGL(flags_kernel, dim3((L + 255) / 256), dim3(256), 0, s, sel, Hkv, nb, L, block, v_radius,
                     v_window, flags);
  ISKV_HIP_CHECK(hipGetLastError());
  return ISKV_OK;
}

size_t iskv_prompt_split_ws_bytes(int32_t L) { return L < 0 ? 0 : ((size_t)L * sizeof(int32_t) + 255) / 256 * 256; }

int iskv_launch_prompt_split(const float* X, const uint8_t* flags, int32_t L, int32_t D, uint32_t mask, int32_t pos0,
                             float* X_keep, int32_t* pos_keep, float* X_rest, int32_t* pos_rest, int32_t* counts,
                             void* ws, hipStream_t s) {
  int32_t* dest = (int32_t*)ws;
  hipLaunchKernelGGL(split_scan_kernel, dim3(1), dim3(1024), 0, s, flags, L, mask, dest, counts);
  if (L > 0)
    hipLaunchKernelGGL(split_gather_kernel, dim3(L), dim3(256), 0, s, X, D, dest, pos0, X_keep, pos_keep, X_rest,
                       pos_rest);
  ISKV_HIP_CHECK(hipGetLastError());
  return ISKV_OK;
}
