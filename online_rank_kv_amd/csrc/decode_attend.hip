// GQA decode attention over a reconstructed cache (iS-KV notes §2.1 and
// Algorithm 3: the model's own dense attention runs on the rebuilt K/V).
// Split-n: each workgroup folds a contiguous chunk of positions for one
// (batch, KV head) into running (max, sum, output) per query head of the
// group; a second kernel merges the chunks with log-sum-exp weights.
#include "iskv_internal.h"

#include <math.h>

#include <mutex>
#include <type_traits>

namespace {

constexpr int DH = 128;

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

// Split kernel: workgroup (split, g, b) folds rows [split * ROWS, +ROWS) of
// KV head g for its G query heads into a partial (max m, sum l, output o).
// Lane l of wave w handles 8 features (chunk l % 16) of row
// w * 32 + 4 i + l / 16 for i = 0..7; all K and V loads of the workgroup are
// issued up front and stay in registers as bf16. Logits reduce over the 16
// lanes of a row; softmax statistics per head over the workgroup's rows;
// P V accumulates per lane and reduces over lanes and waves through LDS.
// Partials layout: part[((b * Hq + h) * nsplit + s) * (DH + 2) + {0: m, 1: l, 2..: o}].
constexpr int ROWS = 128;      // rows per workgroup (4 waves x 32)
constexpr int HG = 4;          // query heads handled per pass

__device__ __forceinline__ void bf8(const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
  f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
  f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
  f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
}

__global__ __launch_bounds__(256) void attend_split_kernel(const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ K,
                                                           const uint16_t* __restrict__ V, int n,
                                                           int Hq, int Hkv, float scale, float* part) {
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int nsplit = gridDim.x;
  const int G = Hq / Hkv;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int c = lane & 15, sr = lane >> 4;
  const int r0 = split * ROWS;
  __shared__ float logit[HG][ROWS];
  __shared__ float red[4][HG][DH];
  __shared__ float stat[HG][2];
  const size_t rstride = (size_t)Hkv * DH;
  const uint16_t* Kb = K + ((size_t)b * n) * rstride + (size_t)g * DH + c * 8;
  const uint16_t* Vb = V + ((size_t)b * n) * rstride + (size_t)g * DH + c * 8;
  uint4 kr[8], vr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = min(r0 + wave * 32 + 4 * i + sr, n - 1);
    kr[i] = *(const uint4*)(Kb + (size_t)row * rstride);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = min(r0 + wave * 32 + 4 * i + sr, n - 1);
    vr[i] = *(const uint4*)(Vb + (size_t)row * rstride);
  }
  for (int h0 = 0; h0 < G; h0 += HG) {
    const int hn = min(HG, G - h0);
    // query chunk of each head of this pass, pre-scaled
    float qf[HG][8];
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      const int h = g * G + h0 + min(hh, hn - 1);
      bf8(*(const uint4*)(q + ((size_t)b * Hq + h) * DH + c * 8), qf[hh]);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[hh][e] *= scale;
    }
    // logits
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float kf[8];
      bf8(kr[i], kf);
      const int rl = wave * 32 + 4 * i + sr;
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(qf[hh][e], kf[e], acc);
        acc += __shfl_xor(acc, 8, 64);
        acc += __shfl_xor(acc, 4, 64);
        acc += __shfl_xor(acc, 2, 64);
        acc += __shfl_xor(acc, 1, 64);
        if (c == 0) logit[hh][rl] = (r0 + rl < n) ? acc : -INFINITY;
      }
    }
    __syncthreads();
    // softmax statistics: wave w handles head w of the pass
    if (wave < hn) {
      float a = logit[wave][lane], bq = logit[wave][lane + 64];
      float m = wave_max(fmaxf(a, bq));
      float pa = (a == -INFINITY) ? 0.f : __expf(a - m);
      float pb = (bq == -INFINITY) ? 0.f : __expf(bq - m);
      float l = wave_sum(pa + pb);
      logit[wave][lane] = pa;
      logit[wave][lane + 64] = pb;
      if (lane == 0) { stat[wave][0] = m; stat[wave][1] = l; }
    }
    __syncthreads();
    // P V
    float acc[HG][8];
#pragma unroll
    for (int hh = 0; hh < HG; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float vf[8];
      bf8(vr[i], vf);
      const int rl = wave * 32 + 4 * i + sr;
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        const float pr = logit[hh][rl];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] = fmaf(pr, vf[e], acc[hh][e]);
      }
    }
    // reduce over the 4 row lanes of each chunk, then over waves
#pragma unroll
    for (int hh = 0; hh < HG; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = acc[hh][e];
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        acc[hh][e] = v;
      }
    if (sr == 0) {
#pragma unroll
      for (int hh = 0; hh < HG; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) red[wave][hh][c * 8 + e] = acc[hh][e];
    }
    __syncthreads();
    for (int idx = t; idx < hn * DH; idx += 256) {
      const int hh = idx / DH, d = idx % DH;
      const float o = red[0][hh][d] + red[1][hh][d] + red[2][hh][d] + red[3][hh][d];
      const int h = g * G + h0 + hh;
      float* dst = part + (((size_t)b * Hq + h) * nsplit + split) * (DH + 2);
      dst[2 + d] = o;
      if (d == 0) { dst[0] = stat[hh][0]; dst[1] = stat[hh][1]; }
    }
    __syncthreads();
  }
}

// Streaming form for GQA groups of up to HG query heads: workgroup
// (split, g, b) folds NCH chunks of 128 rows with an online softmax (running
// max and sum per head, the output rescaled when the max moves) and writes
// one partial per head. Per chunk, lane l
// of wave w holds 8 features (l % 16) of rows w * 32 + 4 i + l / 16 of K and
// of V; the next chunk's K loads are issued once the logits have consumed
// the current K, its V loads once P V has consumed the current V. The 32
// partial dot products of a lane (4 heads x 8 rows) are reduced over the 16
// lanes of a row by recursive halving (30 exchanges instead of 128): lane
// c % 16 ends with the logits of head c / 4 for its rows 2 (c % 4) and
// 2 (c % 4) + 1.
constexpr int CROWS = 128;
template <int NCH>
__global__ __launch_bounds__(256) void attend_stream_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ K,
                                                            const uint16_t* __restrict__ V, int n,
                                                            int Hq, int Hkv, float scale, float* part) {
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int nsplit = gridDim.x;
  const int G = Hq / Hkv;  // 1 .. HG
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int c = lane & 15, sr = lane >> 4;
  const int r0 = split * CROWS * NCH;
  __shared__ float logit[HG][CROWS];
  __shared__ float red[4][HG][DH];
  __shared__ float mrun[HG], lrun[HG], alpha[HG];
  const size_t rstride = (size_t)Hkv * DH;
  const uint16_t* Kb = K + ((size_t)b * n) * rstride + (size_t)g * DH + c * 8;
  const uint16_t* Vb = V + ((size_t)b * n) * rstride + (size_t)g * DH + c * 8;
  uint4 kr[8], vr[8];
  auto load_k = [&](int ch) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = min(r0 + ch * CROWS + wave * 32 + 4 * i + sr, n - 1);
      kr[i] = *(const uint4*)(Kb + (size_t)row * rstride);
    }
  };
  auto load_v = [&](int ch) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = min(r0 + ch * CROWS + wave * 32 + 4 * i + sr, n - 1);
      vr[i] = *(const uint4*)(Vb + (size_t)row * rstride);
    }
  };
  load_k(0);
  load_v(0);
  float qf[HG][8];
#pragma unroll
  for (int hh = 0; hh < HG; ++hh) {
    const int h = g * G + min(hh, G - 1);
    bf8(*(const uint4*)(q + ((size_t)b * Hq + h) * DH + c * 8), qf[hh]);
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[hh][e] *= scale;
  }
  if (t < HG) { mrun[t] = -INFINITY; lrun[t] = 0.f; }
  float acc[HG][8];
#pragma unroll
  for (int hh = 0; hh < HG; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
  const int nch = min(NCH, (n - r0 + CROWS - 1) / CROWS);
  for (int ch = 0; ch < nch; ++ch) {
    // partial logits: v[8 hh + i] = q_hh . k_i over this lane's 8 features
    float v[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float kf[8];
      bf8(kr[i], kf);
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fmaf(qf[hh][e], kf[e], a);
        v[8 * hh + i] = a;
      }
    }
    if (ch + 1 < nch) load_k(ch + 1);
    // recursive halving over the 16 lanes of the row group
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const bool up = (c & 8) != 0;
      const float send = up ? v[j] : v[16 + j];
      v[j] = (up ? v[16 + j] : v[j]) + __shfl_xor(send, 8, 64);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool up = (c & 4) != 0;
      const float send = up ? v[j] : v[8 + j];
      v[j] = (up ? v[8 + j] : v[j]) + __shfl_xor(send, 4, 64);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool up = (c & 2) != 0;
      const float send = up ? v[j] : v[4 + j];
      v[j] = (up ? v[4 + j] : v[j]) + __shfl_xor(send, 2, 64);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bool up = (c & 1) != 0;
      const float send = up ? v[j] : v[2 + j];
      v[j] = (up ? v[2 + j] : v[j]) + __shfl_xor(send, 1, 64);
    }
    {  // v[0], v[1]: head c / 4, rows i = 2 (c % 4) and i + 1
      const int hh = c >> 2, i = 2 * (c & 3);
      const int rl = wave * 32 + 4 * i + sr, rb = r0 + ch * CROWS;
      logit[hh][rl] = (rb + rl < n) ? v[0] : -INFINITY;
      logit[hh][rl + 4] = (rb + rl + 4 < n) ? v[1] : -INFINITY;
    }
    __syncthreads();
    // chunk statistics: wave w updates head w's running max and sum
    if (wave < G && wave < HG) {
      const float a = logit[wave][lane], bq = logit[wave][lane + 64];
      const float mo = mrun[wave];
      const float mn = fmaxf(mo, wave_max(fmaxf(a, bq)));
      const float pa = (a == -INFINITY) ? 0.f : __expf(a - mn);
      const float pb = (bq == -INFINITY) ? 0.f : __expf(bq - mn);
      const float ls = wave_sum(pa + pb);
      logit[wave][lane] = pa;
      logit[wave][lane + 64] = pb;
      if (lane == 0) {
        const float al = (mo == -INFINITY) ? 0.f : __expf(mo - mn);
        alpha[wave] = al;
        mrun[wave] = mn;
        lrun[wave] = lrun[wave] * al + ls;
      }
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      const float al = alpha[hh];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] *= al;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float vf[8];
      bf8(vr[i], vf);
      const int rl = wave * 32 + 4 * i + sr;
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        const float pr = logit[hh][rl];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] = fmaf(pr, vf[e], acc[hh][e]);
      }
    }
    if (ch + 1 < nch) load_v(ch + 1);
    __syncthreads();  // logit and alpha are rewritten by the next chunk
  }
  // reduce over the 4 row lanes of each chunk, then over waves
#pragma unroll
  for (int hh = 0; hh < HG; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = acc[hh][e];
      x += __shfl_xor(x, 16, 64);
      x += __shfl_xor(x, 32, 64);
      acc[hh][e] = x;
    }
  if (sr == 0) {
#pragma unroll
    for (int hh = 0; hh < HG; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave][hh][c * 8 + e] = acc[hh][e];
  }
  __syncthreads();
  for (int idx = t; idx < G * DH; idx += 256) {
    const int hh = idx / DH, d = idx % DH;
    const float o = red[0][hh][d] + red[1][hh][d] + red[2][hh][d] + red[3][hh][d];
    const int h = g * G + hh;
    float* dst = part + (((size_t)b * Hq + h) * nsplit + split) * (DH + 2);
    dst[2 + d] = o;
    if (d == 0) { dst[0] = mrun[hh]; dst[1] = lrun[hh]; }
  }
}

// Combine: one workgroup per (batch, query head). Split weights
// w_s = exp(m_s - M) and L = sum w_s l_s are formed in parallel; each wave
// then sums a quarter of the splits for all 128 features and the quarters are
// added through LDS.
__global__ __launch_bounds__(256) void attend_combine_kernel(const float* __restrict__ part,
                                                             int nsplit, uint16_t* out) {
  const int bh = blockIdx.x;
  const float* src = part + (size_t)bh * nsplit * (DH + 2);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  extern __shared__ float cw[];  // [nsplit] weights
  __shared__ float redm[4], redl[4];
  __shared__ float acc4[4][DH];
  float m = -INFINITY;
  for (int s = t; s < nsplit; s += 256) m = fmaxf(m, src[(size_t)s * (DH + 2)]);
  m = wave_max(m);
  if (lane == 0) redm[wave] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(redm[0], redm[1]), fmaxf(redm[2], redm[3]));
  float l = 0.f;
  for (int s = t; s < nsplit; s += 256) {
    const float ms = src[(size_t)s * (DH + 2)];
    const float w = (ms == -INFINITY) ? 0.f : __expf(ms - M);
    cw[s] = w;
    l += w * src[(size_t)s * (DH + 2) + 1];
  }
  l = wave_sum(l);
  if (lane == 0) redl[wave] = l;
  __syncthreads();
  const float L = redl[0] + redl[1] + redl[2] + redl[3];
  const int per = (nsplit + 3) / 4;
  const int s0 = wave * per, s1 = min(nsplit, s0 + per);
  float a0 = 0.f, a1 = 0.f;
#pragma unroll 8
  for (int s = s0; s < s1; ++s) {
    const float w = cw[s];
    a0 = fmaf(w, src[(size_t)s * (DH + 2) + 2 + lane], a0);
    a1 = fmaf(w, src[(size_t)s * (DH + 2) + 2 + 64 + lane], a1);
  }
  acc4[wave][lane] = a0;
  acc4[wave][lane + 64] = a1;
  __syncthreads();
  if (t < DH) {
    const float o = acc4[0][t] + acc4[1][t] + acc4[2][t] + acc4[3][t];
    out[(size_t)bh * DH + t] = f2bf(o / L);
  }
}

static int num_splits(int n) { return (n + ROWS - 1) / ROWS; }

// Scratch of decode_attend_noalloc: the split kernel's (max, sum, output)
// partials live in this fixed array instead of a caller workspace. Every
// device holds its own copy until the process ends. Host code uses only the
// per-device address from hipGetSymbolAddress, never the array's name.
constexpr size_t ATTEND_SCRATCH_BYTES = (size_t)8 << 20;
__device__ __align__(256) float scratch[ATTEND_SCRATCH_BYTES / sizeof(float)];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[MAX_DEVICES] = {};

// Device address of this device's scratch, looked up once per device with
// that device current.
int scratch_for(int dev, float** out) {
  if (dev < 0 || dev >= MAX_DEVICES) return ISKV_EINVAL;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    ISKV_HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return ISKV_EHIP;
    g_scratch_ptr[dev] = (float*)p;
  }
  *out = g_scratch_ptr[dev];
  return ISKV_OK;
}

}  // namespace

int iskv_launch_attend_noalloc(const uint16_t* q, const uint16_t* K, const uint16_t* V, int32_t batch, int32_t n,
                               int32_t Hq, int32_t Hkv, int32_t dh, float scale, uint16_t* out, hipStream_t s) {
  if (iskv_attend_ws_bytes(batch, n, Hq, dh) > ATTEND_SCRATCH_BYTES) return ISKV_EWORKSPACE;
  int dev = 0;
  ISKV_HIP_CHECK(hipGetDevice(&dev));
  if (s) {  // the stream must belong to the current device
    int sdev = -1;
    ISKV_HIP_CHECK(hipStreamGetDevice(s, &sdev));
    if (sdev != dev) return ISKV_EINVAL;
  }
  float* ws = nullptr;
  const int rc = scratch_for(dev, &ws);
  if (rc) return rc;
  return iskv_launch_attend(q, K, V, batch, n, Hq, Hkv, dh, scale, out, ws, ATTEND_SCRATCH_BYTES, s);
}

size_t iskv_attend_ws_bytes(int32_t batch, int32_t n, int32_t Hq, int32_t dh) {
  (void)dh;
  return (size_t)batch * Hq * num_splits(n) * (DH + 2) * sizeof(float);
}

int iskv_launch_attend(const uint16_t* q, const uint16_t* K, const uint16_t* V, int32_t batch,
                       int32_t n, int32_t Hq, int32_t Hkv, int32_t dh, float scale, uint16_t* out,
                       void* ws, size_t ws_bytes, hipStream_t s) {
  (void)dh;
  if (ws_bytes < iskv_attend_ws_bytes(batch, n, Hq, dh)) return ISKV_EWORKSPACE;
  int ns = num_splits(n);
  if (Hq / Hkv <= HG) {
    // streaming form; chunks of 128 rows per workgroup by length (measured at
    // 8 KV heads: one chunk is fastest up to ~32K rows, where the grid
    // already holds a thousand workgroups; longer caches fold 4 or 8 chunks
    // per workgroup and keep the combine's partials few)
    const int chunks = (n + CROWS - 1) / CROWS;
    auto go = [&](auto nch_c) {
      constexpr int NCH = decltype(nch_c)::value;
      const int nsp = (chunks + NCH - 1) / NCH;
      hipLaunchKernelGGL((attend_stream_kernel<NCH>), dim3(nsp, Hkv, batch), dim3(256), 0, s, q, K, V, n, Hq, Hkv,
                         scale, (float*)ws);
      return nsp;
    };
    ns = chunks <= 256 ? go(std::integral_constant<int, 1>{})
                       : (chunks <= 1024 ? go(std::integral_constant<int, 4>{}) : go(std::integral_constant<int, 8>{}));
  } else {
    hipLaunchKernelGGL(attend_split_kernel, dim3(ns, Hkv, batch), dim3(256), 0, s, q, K, V, n, Hq, Hkv,
                       scale, (float*)ws);
  }
  hipLaunchKernelGGL(attend_combine_kernel, dim3(batch * Hq), dim3(256), (size_t)ns * sizeof(float), s,
                     (const float*)ws, ns, out);
  ISKV_HIP_CHECK(hipGetLastError());
  return ISKV_OK;
}
