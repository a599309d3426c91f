// GQA decode attention over a reconstructed cache (iS-KV notes §2.1 and
// Algorithm 3: the model's own dense attention runs on the rebuilt K/V).
// Split-n: each workgroup folds a contiguous chunk of positions for one
// (batch, KV head) into running (max, sum, output) per query head of the
// group; a second kernel merges the chunks with log-sum-exp weights.
#include "iskv_internal.h"

#include <math.h>

namespace {

constexpr int DH = 128;
constexpr int TILE = 64;
constexpr int MAXG = 16;

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Partials layout: part[((b * Hq + h) * nsplit + s) * (DH + 2) + {0: m, 1: l, 2..: o}].
__global__ __launch_bounds__(256) void attend_split_kernel(const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ K,
                                                           const uint16_t* __restrict__ V, int n,
                                                           int Hq, int Hkv, float scale,
                                                           int rows_per_split, float* part) {
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int nsplit = gridDim.x;
  const int G = Hq / Hkv;
  __shared__ float Ks[TILE][DH + 1];
  __shared__ float Vs[TILE][DH];
  __shared__ float qs[MAXG][DH];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int idx = t; idx < G * DH; idx += 256) {
    int hh = idx / DH, c = idx % DH;
    qs[hh][c] = bf2f(q[((size_t)b * Hq + g * G + hh) * DH + c]) * scale;
  }
  const int r0 = split * rows_per_split;
  const int r1 = min(n, r0 + rows_per_split);
  // per-wave running state for heads wave, wave+4, ... (at most 4 per wave)
  float m_run[MAXG / 4], l_run[MAXG / 4], o0[MAXG / 4], o1[MAXG / 4];
#pragma unroll
  for (int u = 0; u < MAXG / 4; ++u) { m_run[u] = -INFINITY; l_run[u] = 0.f; o0[u] = 0.f; o1[u] = 0.f; }
  const size_t rstride = (size_t)Hkv * DH;
  const uint16_t* Kb = K + ((size_t)b * n) * rstride + (size_t)g * DH;
  const uint16_t* Vb = V + ((size_t)b * n) * rstride + (size_t)g * DH;
  for (int tr = r0; tr < r1; tr += TILE) {
    __syncthreads();
    // 64 rows x 16 chunks of 8 bf16
    for (int idx = t; idx < TILE * 16; idx += 256) {
      int rr = idx >> 4, ch = idx & 15;
      int row = tr + rr;
      if (row < r1) {
        uint4 kv = *(const uint4*)(Kb + (size_t)row * rstride + ch * 8);
        uint4 vv = *(const uint4*)(Vb + (size_t)row * rstride + ch * 8);
        const uint16_t* kp = (const uint16_t*)&kv;
        const uint16_t* vp = (const uint16_t*)&vv;
#pragma unroll
        for (int e = 0; e < 8; ++e) { Ks[rr][ch * 8 + e] = bf2f(kp[e]); Vs[rr][ch * 8 + e] = bf2f(vp[e]); }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) { Ks[rr][ch * 8 + e] = 0.f; Vs[rr][ch * 8 + e] = 0.f; }
      }
    }
    __syncthreads();
    const int row = tr + lane;
#pragma unroll
    for (int u = 0; u < MAXG / 4; ++u) {
      const int hh = wave + 4 * u;
      if (hh >= G) break;
      float logit = -INFINITY;
      if (row < r1) {
        float acc = 0.f;
#pragma unroll 16
        for (int c = 0; c < DH; ++c) acc = fmaf(qs[hh][c], Ks[lane][c], acc);
        logit = acc;
      }
      float mt = wave_max(logit);
      float mnew = fmaxf(m_run[u], mt);
      float p = (row < r1) ? __expf(logit - mnew) : 0.f;
      float alpha = (m_run[u] == -INFINITY) ? 0.f : __expf(m_run[u] - mnew);
      l_run[u] = l_run[u] * alpha + wave_sum(p);
      float a0 = o0[u] * alpha, a1 = o1[u] * alpha;
      for (int rr = 0; rr < TILE; ++rr) {
        float pr = __shfl(p, rr, 64);
        a0 = fmaf(pr, Vs[rr][lane], a0);
        a1 = fmaf(pr, Vs[rr][lane + 64], a1);
      }
      o0[u] = a0; o1[u] = a1;
      m_run[u] = mnew;
    }
  }
#pragma unroll
  for (int u = 0; u < MAXG / 4; ++u) {
    const int hh = wave + 4 * u;
    if (hh >= G) break;
    const int h = g * G + hh;
    float* dst = part + (((size_t)b * Hq + h) * nsplit + split) * (DH + 2);
    if (lane == 0) { dst[0] = m_run[u]; dst[1] = l_run[u]; }
    dst[2 + lane] = o0[u];
    dst[2 + lane + 64] = o1[u];
  }
}

__global__ __launch_bounds__(128) void attend_combine_kernel(const float* __restrict__ part,
                                                             int nsplit, uint16_t* out) {
  const int bh = blockIdx.x;
  const float* src = part + (size_t)bh * nsplit * (DH + 2);
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, src[s * (DH + 2)]);
  float L = 0.f, acc = 0.f;
  const int c = threadIdx.x;
  for (int s = 0; s < nsplit; ++s) {
    float ms = src[s * (DH + 2)];
    if (ms == -INFINITY) continue;
    float w = __expf(ms - M);
    L += w * src[s * (DH + 2) + 1];
    acc += w * src[s * (DH + 2) + 2 + c];
  }
  out[(size_t)bh * DH + c] = f2bf(acc / L);
}

static int pick_splits(int batch, int n, int Hkv) {
  int tiles = (n + TILE - 1) / TILE;
  int want = (2048 + batch * Hkv - 1) / (batch * Hkv);
  int ns = tiles < want ? tiles : want;
  return ns < 1 ? 1 : ns;
}

}  // namespace

size_t iskv_attend_ws_bytes(int32_t batch, int32_t n, int32_t Hq, int32_t dh) {
  (void)dh;
  int ns = pick_splits(batch, n, 1);
  return (size_t)batch * Hq * ns * (DH + 2) * sizeof(float);
}

int iskv_launch_attend(const uint16_t* q, const uint16_t* K, const uint16_t* V, int32_t batch,
                       int32_t n, int32_t Hq, int32_t Hkv, int32_t dh, float scale, uint16_t* out,
                       void* ws, size_t ws_bytes, hipStream_t s) {
  (void)dh;
  int ns = pick_splits(batch, n, Hkv);
  size_t need = (size_t)batch * Hq * ns * (DH + 2) * sizeof(float);
  if (ws_bytes < need) return ISKV_EWORKSPACE;
  int tiles = (n + TILE - 1) / TILE;
  int tiles_per = (tiles + ns - 1) / ns;
  int rows_per = tiles_per * TILE;
  ns = (n + rows_per - 1) / rows_per;
  hipLaunchKernelGGL(attend_split_kernel, dim3(ns, Hkv, batch), dim3(256), 0, s, q, K, V, n, Hq, Hkv,
                     scale, rows_per, (float*)ws);
  hipLaunchKernelGGL(attend_combine_kernel, dim3(batch * Hq), dim3(128), 0, s, (const float*)ws, ns,
                     out);
  ISKV_HIP_CHECK(hipGetLastError());
  return ISKV_OK;
}
