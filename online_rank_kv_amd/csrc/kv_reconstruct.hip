// Reconstruction of the dense KV cache from the factors, with per-position
// RoPE on keys, and the exact-row scatter (iS-KV notes §3.2, §5.2,
// Algorithm 3). Output row t holds the token at original position t.
#include "iskv_internal.h"

#include <math.h>

#include <type_traits>

namespace {

__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <bool BF16>
__device__ __forceinline__ void store_out(void* out, size_t idx, float v) {
  if (BF16) ((uint16_t*)out)[idx] = f2bf(v);
  else ((float*)out)[idx] = v;
}

// Angle of rotary pair j at position pos: pos * theta^(-2j/dh), formed and
// reduced modulo 2 pi in fp64 so that positions in the tens of thousands keep
// fp32-level accuracy, then sin/cos of the reduced fp32 angle.
__device__ __forceinline__ void rope_cs(int pos, double inv_freq, float* c, float* s) {
  const double two_pi = 6.283185307179586476925286766559;
  double phi = (double)pos * inv_freq;
  double red = phi - two_pi * rint(phi / two_pi);
  sincosf((float)red, s, c);
}

// Two fp32 values to packed bf16 (round to nearest even) with one
// v_cvt_pk_bf16_f32.
typedef float f2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{a, b}, bf2_t));
}

// RoPE angle in revolutions for the bf16 paths: f = theta^(-2j/dh) / (2 pi)
// is held as a 64-bit binary fraction F (f < 1/2); the fractional part of
// pos * f is then the top 32 bits of pos * F mod 2^64, read as a signed
// fraction in [-1/2, 1/2). Exact integer arithmetic: the only errors are F's
// rounding (2^-54 relative) and the final 2^-32 truncation, for any position
// below 2^31.
__device__ __forceinline__ uint64_t rope_fraction(double rev_per_pos) {
  return (uint64_t)(rev_per_pos * 18446744073709551616.0);  // * 2^64
}
__device__ __forceinline__ float rope_rev(uint32_t p, uint64_t F) {
  const uint32_t flo = (uint32_t)F, fhi = (uint32_t)(F >> 32);
  const uint32_t top = p * fhi + __umulhi(p, flo);
  return (float)(int32_t)top * 2.3283064365386963e-10f;  // * 2^-32
}

// Four consecutive stored coordinates as fp32 (fp32 rows, or bf16 / fp16 rows
// under 2-byte persistence; the 2-byte loads need 8-byte alignment).
__device__ __forceinline__ float4 ld_c4(const float* p) { return *(const float4*)p; }
__device__ __forceinline__ float4 ld_c4(const uint16_t* p) {
  const uint2 v = *(const uint2*)p;
  return float4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
                __uint_as_float(v.y & 0xffff0000u)};
}
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float4 ld_c4(const _Float16* p) {
  const uint2 v = *(const uint2*)p;
  const h2_t a = __builtin_bit_cast(h2_t, v.x), b = __builtin_bit_cast(h2_t, v.y);
  return float4{(float)a.x, (float)a.y, (float)b.x, (float)b.y};
}

// Column tile of W (128 or 64) features; rotary pair q (0 .. W/2-1) of the
// tile is (lo, lo + dh/2) with lo = (q / (dh/2)) * dh + q % (dh/2).
// Requires W % dh == 0.
__device__ __forceinline__ int pair_lo(int q, int dh) {
  const int half = dh >> 1;
  return (q / half) * dh + (q % half);
}

// Compressed rows: out[pos[i], tile] = RoPE(C[i, :k] B[tile, :k]^T).
// Grid (D / W, ceil(n / 32)); 256 threads; thread owns 4 rows x 2 pairs
// (one pair when W == 64).
template <bool BF16, typename TC>
__global__ __launch_bounds__(256) void recon_kernel(const TC* __restrict__ C, int ldc,
                                                    const float* __restrict__ B, int ldb,
                                                    const int32_t* __restrict__ pos,
                                                    const int32_t* __restrict__ st, int n, int D,
                                                    int dh, int W, int apply_rope,
                                                    double log_theta, void* out, int n_total) {
  const int k = st[ST_K];
  const int c0 = blockIdx.x * W;
  const int i0 = blockIdx.y * 32;
  if (i0 >= n) return;
  __shared__ float Cs[32][33];
  __shared__ float Bs[128][33];
  const int t = threadIdx.x;
  const int rg = (t >> 5) * 4;       // rows rg .. rg+3
  const int q0 = t & 31;
  const bool two = W == 128;
  const int q1 = two ? q0 + 32 : q0;
  const int lo0 = pair_lo(q0, dh), hi0 = lo0 + dh / 2;
  const int lo1 = pair_lo(q1, dh), hi1 = lo1 + dh / 2;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < k; k0 += 32) {
    for (int idx = t; idx < 32 * 32; idx += 256) {
      int r = idx >> 5, c = idx & 31;
      Cs[r][c] = (i0 + r < n && k0 + c < k) ? iskv_ld(C + (size_t)(i0 + r) * ldc + k0 + c) : 0.f;
    }
    for (int idx = t; idx < W * 32; idx += 256) {
      int r = idx >> 5, c = idx & 31;
      Bs[r][c] = (k0 + c < k) ? B[(size_t)(c0 + r) * ldb + k0 + c] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk) {
      float b0 = Bs[lo0][kk], b1 = Bs[hi0][kk], b2 = Bs[lo1][kk], b3 = Bs[hi1][kk];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float a = Cs[rg + u][kk];
        acc[u][0] = fmaf(a, b0, acc[u][0]);
        acc[u][1] = fmaf(a, b1, acc[u][1]);
        acc[u][2] = fmaf(a, b2, acc[u][2]);
        acc[u][3] = fmaf(a, b3, acc[u][3]);
      }
    }
    __syncthreads();
  }
  const int half = dh / 2;
  const double inv0 = exp(-(2.0 * (q0 % half) / dh) * log_theta);
  const double inv1 = exp(-(2.0 * (q1 % half) / dh) * log_theta);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    int i = i0 + rg + u;
    if (i >= n) continue;
    int p = pos[i];
    if (p < 0 || p >= n_total) continue;  // outside the output: dropped, never written
    float x0 = acc[u][0], y0 = acc[u][1], x1 = acc[u][2], y1 = acc[u][3];
    if (apply_rope) {
      float c, s;
      rope_cs(p, inv0, &c, &s);
      float a0 = x0 * c - y0 * s, b0 = y0 * c + x0 * s;
      rope_cs(p, inv1, &c, &s);
      float a1 = x1 * c - y1 * s, b1 = y1 * c + x1 * s;
      x0 = a0; y0 = b0; x1 = a1; y1 = b1;
    }
    size_t base = (size_t)p * D + c0;
    store_out<BF16>(out, base + lo0, x0);
    store_out<BF16>(out, base + hi0, y0);
    if (two) {
      store_out<BF16>(out, base + lo1, x1);
      store_out<BF16>(out, base + hi1, y1);
    }
  }
}

// bf16 MFMA reconstruction of the compressed rows (bf16 output):
// out[pos[i], c0 .. c0+127] = RoPE(C[i, :k] B[c0 .. c0+127, :k]^T).
// C (fp32) is rounded to bf16 while it is staged, B comes from its bf16 copy;
// products accumulate in fp32 (v_mfma_f32_16x16x32_bf16).
// Workgroup: 64 rows x 128 features, 4 waves; wave (wr, wc) owns rows
// wr*32 .. +31 and four 16-feature blocks: two "lo" blocks and the blocks
// half a head further, so both members of every rotary pair (j, j + dh/2)
// sit in the same lane and accumulator element and RoPE is applied in
// registers. Workgroup w maps to row block g*8 + w%8 and feature tile
// (w / 8) % T, with g = w / (8T): the T feature tiles of one row block are
// dispatched to the same XCD and share its L2 copy of the C rows.
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
constexpr int RM_BM = 64, RM_BN = 128, RM_KC = 64;
constexpr int RM_RS = RM_KC + 8;    // LDS row stride (bf16) of the staged operands
constexpr int RM_OS = RM_BN + 8;    // LDS row stride (bf16) of the output tile
constexpr int RM_LDS = (RM_BM + RM_BN) * RM_RS;  // bf16 elements
static_assert(RM_BM * RM_OS <= RM_LDS, "output tile must fit in the staging area");

template <typename TC>
__global__ __launch_bounds__(256) void recon_mfma_kernel(const TC* __restrict__ C, int ldc,
                                                         const uint16_t* __restrict__ Bbf, int ldb,
                                                         const int32_t* __restrict__ pos,
                                                         const int32_t* __restrict__ st, int n,
                                                         int D, int dh, int apply_rope,
                                                         double log_theta, uint16_t* out,
                                                         int n_total, int tiles) {
  const int k = st[ST_K];
  const int w = blockIdx.x;
  const int g = w / (8 * tiles), rem = w % (8 * tiles);
  const int i0 = (g * 8 + rem % 8) * RM_BM, c0 = (rem / 8) * RM_BN;
  if (i0 >= n) return;
  __shared__ __attribute__((aligned(16))) uint16_t lds[RM_LDS];
  uint16_t* Cs = lds;                  // [64][RM_RS]   C rows, k chunk
  uint16_t* Bs = lds + RM_BM * RM_RS;  // [128][RM_RS]  B rows (features), k chunk
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int half = dh >> 1;
  // the tile's "lo" 16-feature blocks in order; this wave takes two of them
  int lob0 = 0, lob1 = 0;
  {
    int cnt = 0;
    for (int b = 0; b < RM_BN / 16; ++b) {
      if ((b * 16) % dh < half) {
        if (cnt == 2 * wc) lob0 = b;
        if (cnt == 2 * wc + 1) lob1 = b;
        ++cnt;
      }
    }
  }
  const int blk[4] = {lob0, lob1, lob0 + half / 16, lob1 + half / 16};
  v4f acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < k; k0 += RM_KC) {
    if (k0 > 0) __syncthreads();
    // C: 64 x 64 fp32 -> bf16; columns >= k (and rows >= n) are zero
    float4 cv[4];
    uint4 bv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int e = t + 256 * u, r = e >> 4, col = k0 + (e & 15) * 4;
      int row = min(i0 + r, n - 1), colc = min(col, ldc - 4);
      cv[u] = ld_c4(C + (size_t)row * ldc + colc);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int e = t + 256 * u, r = e >> 3, col = k0 + (e & 7) * 8;
      int colc = min(col, ldb - 8);
      bv[u] = *(const uint4*)(Bbf + (size_t)(c0 + r) * ldb + colc);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int e = t + 256 * u, r = e >> 4, cl = (e & 15) * 4, col = k0 + cl;
      float x0 = col < k ? cv[u].x : 0.f, x1 = col + 1 < k ? cv[u].y : 0.f;
      float x2 = col + 2 < k ? cv[u].z : 0.f, x3 = col + 3 < k ? cv[u].w : 0.f;
      uint2 pk;
      pk.x = (uint32_t)f2bf(x0) | ((uint32_t)f2bf(x1) << 16);
      pk.y = (uint32_t)f2bf(x2) | ((uint32_t)f2bf(x3) << 16);
      *(uint2*)(Cs + r * RM_RS + cl) = pk;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int e = t + 256 * u, r = e >> 3, cl = (e & 7) * 8, col = k0 + cl;
      uint4 v = bv[u];
      if (col + 8 > k) {  // partial chunk at the rank boundary: zero k >= rank
        uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (col + q >= k) wv[q >> 1] &= (q & 1) ? 0x0000ffffu : 0xffff0000u;
        v = uint4{wv[0], wv[1], wv[2], wv[3]};
      }
      *(uint4*)(Bs + r * RM_RS + cl) = v;
    }
    __syncthreads();
    // A operand: lane holds C(row l%16, k 8(l/16) .. +7); B operand: lane
    // holds B(feature l%16, same k range)
#pragma unroll
    for (int ks = 0; ks < RM_KC; ks += 32) {
      const int ko = ks + 8 * (lane >> 4);
      v8bf a0 = __builtin_bit_cast(v8bf, *(const uint4*)(Cs + (wr * 32 + (lane & 15)) * RM_RS + ko));
      v8bf a1 = __builtin_bit_cast(v8bf, *(const uint4*)(Cs + (wr * 32 + 16 + (lane & 15)) * RM_RS + ko));
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        v8bf bb = __builtin_bit_cast(v8bf, *(const uint4*)(Bs + (blk[b] * 16 + (lane & 15)) * RM_RS + ko));
        acc[0][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bb, acc[0][b], 0, 0, 0);
        acc[1][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bb, acc[1][b], 0, 0, 0);
      }
    }
  }
  __syncthreads();
  // epilogue: lane l, element e holds row 4(l/16) + e, feature l%16 of each block.
  // RoPE: the angle pos * theta^(-2j/dh) is formed in revolutions in fp64 and
  // reduced to [-1/2, 1/2]; sin and cos of the reduced fp32 value (the
  // hardware sine/cosine take revolutions) are far below bf16 resolution.
  uint16_t* Os = lds;  // [64][RM_OS] output tile
  double rev_per_pos[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int j = (blk[b] * 16 + (lane & 15)) % dh;
    rev_per_pos[b] = exp(-(2.0 * j / dh) * log_theta) * 0.15915494309189533577;  // / (2 pi)
  }
#pragma unroll
  for (int a = 0; a < 2; ++a) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int rl = wr * 32 + a * 16 + 4 * (lane >> 4) + e;
      const int i = i0 + rl;
      const int p = pos[min(i, n - 1)];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        float x = acc[a][b][e], y = acc[a][b + 2][e];
        const int flo = blk[b] * 16 + (lane & 15);
        if (apply_rope) {
          double rv = (double)p * rev_per_pos[b];
          float r = (float)(rv - rint(rv));
          float c = __builtin_amdgcn_cosf(r), s = __builtin_amdgcn_sinf(r);
          float xr = x * c - y * s, yr = y * c + x * s;
          x = xr; y = yr;
        }
        Os[rl * RM_OS + flo] = f2bf(x);
        Os[rl * RM_OS + flo + half] = f2bf(y);
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    int e = t + 256 * u, r = e >> 4, cl = (e & 15) * 8;
    int i = i0 + r;
    if (i >= n) continue;
    int p = pos[i];
    if (p < 0 || p >= n_total) continue;  // outside the output: dropped, never written
    *(uint4*)(out + (size_t)p * D + c0 + cl) = *(const uint4*)(Os + r * RM_OS + cl);
  }
}

// Streaming form of the bf16 MFMA reconstruction for k <= 256 (r_max a
// multiple of 32, at most 256): each workgroup keeps one 128-feature tile of
// B^T in registers for the whole launch (wave w holds the MFMA B operands of
// its two 16-feature blocks, the "lo" block and the one half a head further,
// for every k step) and streams 32-row blocks of C through LDS: the loads of
// the block two ahead are in flight while the current block is multiplied.
// The product is taken transposed, out^T = B C^T (B as the MFMA's left
// operand), so that lane l holds four consecutive features of token l % 16
// for both members of each rotary pair: it rotates them in registers and
// stores 8 bytes per member straight into the token's row (neighbouring
// lanes and waves fill the rest of the row's 256 bytes). One barrier per
// block: the two staging buffers alternate. Workgroup w serves feature tile (w / 8) % T and row blocks
// rs, rs + S, ... with rs = w % 8 + 8 (w / 8T): the T tiles of a row block run
// on the same XCD and share its L2 copy of the C rows.
// Memory operations are issued so that the hardware's in-order counter can
// wait for exactly the block in use: every block issues the same eight C
// loads (a block past the end reads through an empty buffer descriptor:
// zeros, no memory traffic) and the same two stores (rows without a valid
// position are sent past the end of the output descriptor, which drops
// them), and the row positions of 16 blocks at a time are staged in LDS
// beforehand, so no per-block load waits behind the prefetches and stores.
constexpr int RS_BM32 = 32;          // rows per block of the 4-wave form
// One history's compressed rows for the streaming kernel: coordinates (TC,
// leading dimension r_max), its bf16 basis copy, row positions, state words
// (k), bf16 output cache [n_total x D], row count and RoPE switch. Several
// histories of one configuration go in one launch.
struct RsPath {
  const void* C;
  const uint16_t* Bbf;
  const int32_t* pos;
  const int32_t* st;
  uint16_t* out;
  int32_t n, n_total, rope, pad;
};
struct RsPaths {
  RsPath p[ISKV_RECON_MAX_PATHS];
};
constexpr int RS_PCH = 16;           // blocks whose positions are staged at once

template <typename TC, int NW, int RS_BM, int KC>  // NW waves: a tile of 32 NW features; RS_BM rows per block;
                                                   // KC: staged columns of C (r_max <= KC: 256 or 512)
__global__ __launch_bounds__(64 * NW, 2) void recon_stream_kernel(const RsPaths paths, int np,
                                                           int ldc, int ldb, int D, int dh, double log_theta,
                                                           int T, int S_all) {
  constexpr int NT = 64 * NW;          // threads
  constexpr int CQ = KC / 4;           // 4-coordinate groups per staged row
  constexpr int KS = KC / 32;          // 32-deep MFMA steps
  constexpr int CS = KC + 8;           // LDS row stride (bf16) of a staged C block
  constexpr int PER = RS_BM * CQ / NT; // float4 (or 4-coordinate) loads per thread per block
  const int wg = blockIdx.x;
  const int ct = (wg / 8) % T, rs_all = wg % 8 + 8 * (wg / (8 * T));
  // row group rs_all serves path rs_all % np as its (rs_all / np)-th of S
  // row groups (consecutive row groups alternate paths)
  const int path = rs_all % np, rs = rs_all / np, S = (S_all - path + np - 1) / np;
  const TC* __restrict__ C = (const TC*)paths.p[path].C;
  const uint16_t* __restrict__ Bbf = paths.p[path].Bbf;
  const int32_t* __restrict__ pos = paths.p[path].pos;
  uint16_t* out = paths.p[path].out;
  const int n = paths.p[path].n, n_total = paths.p[path].n_total, apply_rope = paths.p[path].rope;
  const int kdev = paths.p[path].st[ST_K];
  const int c0 = ct * 32 * NW;
  const int nblk = (n + RS_BM - 1) / RS_BM;
  if (rs >= nblk) return;
  __shared__ __attribute__((aligned(16))) uint16_t Cs[2][RS_BM * CS];
  __shared__ int posC[RS_PCH * RS_BM];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int half = dh >> 1;
  const int ks = (kdev + 31) / 32;
  // this wave's "lo" block (the wave-th block with (16 b) % dh < dh/2) and its partner
  int lob = 0;
  {
    int cnt = 0;
    for (int b = 0; b < 2 * NW; ++b)
      if ((b * 16) % dh < half) {
        if (cnt == wave) lob = b;
        ++cnt;
      }
  }
  const int blk0 = lob, blk1 = lob + half / 16;
  // left MFMA operands: lane holds B(feature 16 blk + l%16, k 32 s + 8 (l/16) .. +7)
  uint4 breg[2][KS];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int f = c0 + 16 * (cb ? blk1 : blk0) + (lane & 15);
#pragma unroll
    for (int sk = 0; sk < KS; ++sk) {
      const int kk = 32 * sk + 8 * (lane >> 4);
      uint4 v = *(const uint4*)(Bbf + (size_t)f * ldb + min(kk, ldb - 8));
      if (kk + 8 > kdev) {  // zero depths >= k
        uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (kk + q >= kdev) wv[q >> 1] &= (q & 1) ? 0x0000ffffu : 0xffff0000u;
        v = uint4{wv[0], wv[1], wv[2], wv[3]};
      }
      breg[cb][sk] = v;
    }
  }
  // tile-local features of this lane's lo members: 16 blk0 + 4 (l / 16) + e
  const int flo = 16 * blk0 + 4 * (lane >> 4);
  uint64_t rope_F[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    rope_F[e] = rope_fraction(exp(-(2.0 * ((flo + e) % dh) / dh) * log_theta) * 0.15915494309189533577);
  // C block staging: element u of this thread is row (t + NT u) / CQ,
  // columns 4 ((t + NT u) % CQ) .. +3. Loads run two blocks ahead (a ring
  // of two register sets).
  constexpr int ES = (int)sizeof(TC);  // bytes per stored coordinate
  // fp32 rows are held as float4, 2-byte rows as their raw bf16 bits
  using CR = std::conditional_t<ES == 4, float4, uint2>;
  CR creg[2][PER];
  // four 2-byte coordinates as bf16 bits (fp16 rows are rounded to bf16)
  auto to_bf4 = [](uint2 v) -> uint2 {
    if constexpr (std::is_same<TC, _Float16>::value) {
      const h2_t a = __builtin_bit_cast(h2_t, v.x), b = __builtin_bit_cast(h2_t, v.y);
      return uint2{pk_bf16((float)a.x, (float)a.y), pk_bf16((float)b.x, (float)b.y)};
    } else {
      return v;
    }
  };
  // C rows through a buffer descriptor based at the block's first row and
  // bounded by the last row n - 1 (rows past n read as zero; a block past the
  // end gets an empty descriptor); per-load offsets are fixed (row t / CQ +
  // (NT / CQ) u, column 4 (t % CQ)), so no address arithmetic runs per block.
  const uint32_t voff0 = (uint32_t)(((t / CQ) * ldc + (t % CQ) * 4) * ES);
  const uint32_t vstep = (uint32_t)((NT / CQ) * ldc * ES);
  auto load_c = [&](int slot, int blk) {
    const bool live = blk < nblk;
    const int i0 = (live ? blk : 0) * RS_BM;
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(C + (size_t)i0 * ldc), (short)0, live ? (int)((n - i0) * ldc * ES) : 0, 0x00020000);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      if constexpr (ES == 4)
        creg[slot][u] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rc, voff0 + u * vstep, 0, 0));
      else
        creg[slot][u] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rc, voff0 + u * vstep, 0, 0));
    }
  };
  // output through one descriptor over the whole cache (n_total x D bf16);
  // an invalid row's offset lies past its end
  const __amdgpu_buffer_rsrc_t ro =
      __builtin_amdgcn_make_buffer_rsrc((void*)out, (short)0, (int)((size_t)n_total * D * 2), 0x00020000);
  auto store_c = [&](int slot, uint16_t* cs, int blk) {
    const int i0 = blk * RS_BM;
    if (i0 + RS_BM <= n && kdev >= ldc) {  // full block: nothing to mask
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int e = t + NT * u, r = e / CQ, c4 = (e % CQ) * 4;
        if constexpr (ES == 4) {
          const float4 v = creg[slot][u];
          *(uint2*)(cs + r * CS + c4) = uint2{pk_bf16(v.x, v.y), pk_bf16(v.z, v.w)};
        } else {
          *(uint2*)(cs + r * CS + c4) = to_bf4(creg[slot][u]);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int e = t + NT * u, r = e / CQ, c4 = (e % CQ) * 4;
        const bool rv = i0 + r < n;
        if constexpr (ES == 4) {
          const float4 v = creg[slot][u];
          const float x0 = (rv && c4 < kdev) ? v.x : 0.f, x1 = (rv && c4 + 1 < kdev) ? v.y : 0.f;
          const float x2 = (rv && c4 + 2 < kdev) ? v.z : 0.f, x3 = (rv && c4 + 3 < kdev) ? v.w : 0.f;
          *(uint2*)(cs + r * CS + c4) = uint2{pk_bf16(x0, x1), pk_bf16(x2, x3)};
        } else {  // zero the 16-bit halves at columns >= k (rows past n read as zero)
          const uint2 v = to_bf4(creg[slot][u]);
          const uint32_t m0 = (c4 < kdev ? 0xffffu : 0u) | (c4 + 1 < kdev ? 0xffff0000u : 0u);
          const uint32_t m1 = (c4 + 2 < kdev ? 0xffffu : 0u) | (c4 + 3 < kdev ? 0xffff0000u : 0u);
          *(uint2*)(cs + r * CS + c4) = rv ? uint2{v.x & m0, v.y & m1} : uint2{0u, 0u};
        }
      }
    }
  };
  // one block through the pipeline; `slot` is a compile-time constant at each
  // call, so the register ring is never indexed at run time. jl: the block's
  // index in the staged position chunk.
  auto process = [&](auto slot_c, int blk, int jl) {
    constexpr int slot = decltype(slot_c)::value;
    uint16_t* cs = Cs[slot];
    const int* ps = posC + jl * RS_BM;
    store_c(slot, cs, blk);
    __syncthreads();
    load_c(slot, blk + 2 * S);
    constexpr int RT = RS_BM / 16;  // 16-token tiles per block
    v4f acc[RT][2];
#pragma unroll
    for (int a = 0; a < RT; ++a)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) acc[a][cb] = v4f{0.f, 0.f, 0.f, 0.f};
    auto kstep = [&](int sk) {
      const int ko = 32 * sk + 8 * (lane >> 4);
#pragma unroll
      for (int a = 0; a < RT; ++a) {
        const v8bf av = __builtin_bit_cast(v8bf, *(const uint4*)(cs + (16 * a + (lane & 15)) * CS + ko));
        acc[a][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, breg[0][sk]), av,
                                                            acc[a][0], 0, 0, 0);
        acc[a][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, breg[1][sk]), av,
                                                            acc[a][1], 0, 0, 0);
      }
    };
    if (ks == KS) {  // the whole rank: no branch between the steps, reads issued ahead
#pragma unroll
      for (int sk = 0; sk < KS; ++sk) kstep(sk);
    } else {
#pragma unroll
      for (int sk = 0; sk < KS; ++sk)
        if (sk < ks) kstep(sk);
    }
    // epilogue: lane l, element e of acc[a][cb] holds feature 4 (l/16) + e of
    // block cb for token 16 a + l % 16
#pragma unroll
    for (int a = 0; a < RT; ++a) {
      const int p = ps[16 * a + (lane & 15)];
      float x[4], y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = acc[a][0][e];
        y[e] = acc[a][1][e];
        if (apply_rope) {
          const float rr = rope_rev((uint32_t)p, rope_F[e]);
          const float c = __builtin_amdgcn_cosf(rr), sn = __builtin_amdgcn_sinf(rr);
          const float xr = x[e] * c - y[e] * sn, yr = y[e] * c + x[e] * sn;
          x[e] = xr; y[e] = yr;
        }
      }
      // rows past n (position -1) and positions outside the output: dropped
      const uint32_t off = (p >= 0 && p < n_total) ? (uint32_t)(((size_t)p * D + c0 + flo) * 2) : 0x80000000u;
      const uint32_t offh = (p >= 0 && p < n_total) ? off + (uint32_t)(half * 2) : 0x80000000u;
      __builtin_amdgcn_raw_buffer_store_b64(v2u{pk_bf16(x[0], x[1]), pk_bf16(x[2], x[3])}, ro, off, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b64(v2u{pk_bf16(y[0], y[1]), pk_bf16(y[2], y[3])}, ro, offh, 0, 0);
    }
  };
  // positions of this workgroup's blocks j0 .. j0 + RS_PCH - 1 (past n: -1)
  auto stage_pos = [&](int j0) {
    __syncthreads();  // the previous chunk's last stores have read it
    for (int e = t; e < RS_PCH * RS_BM; e += NT) {
      const int i = (rs + (j0 + e / RS_BM) * S) * RS_BM + e % RS_BM;
      posC[e] = i < n ? pos[min(i, n - 1)] : -1;
    }
    __syncthreads();
  };
  // this workgroup's blocks in chunks of RS_PCH, each chunk as pairs of
  // blocks with straight-line bodies (an odd last block runs empty: zeros in,
  // nothing stored)
  const int nbw = (nblk - rs + S - 1) / S;
  load_c(0, rs);
  load_c(1, rs + S);
  for (int j0 = 0; j0 < nbw; j0 += RS_PCH) {
    stage_pos(j0);
    const int npair = (min(RS_PCH, nbw - j0) + 1) / 2;
    for (int jp = 0; jp < npair; ++jp) {
      const int b0 = rs + (j0 + 2 * jp) * S;
      process(std::integral_constant<int, 0>{}, b0, 2 * jp);
      process(std::integral_constant<int, 1>{}, b0 + S, 2 * jp + 1);
    }
  }
}

// Exact rows: out[pos_e] = RoPE(X_exact[e]); slots with pos_e < 0 are empty.
// Grid (n_exact), 64 threads x pairs.
template <bool BF16>
__global__ __launch_bounds__(256) void exact_rows_kernel(const float* __restrict__ X,
                                                         const int32_t* __restrict__ pe, int D,
                                                         int dh, int apply_rope, double log_theta,
                                                         void* out, int n_total) {
  const int e = blockIdx.x;
  const int p = pe[e];
  if (p < 0 || p >= n_total) return;
  const int half = dh / 2;
  for (int q = threadIdx.x; q < D / 2; q += blockDim.x) {
    int head = q / half, j = q % half;
    int lo = head * dh + j, hi = lo + half;
    float x = X[(size_t)e * D + lo], y = X[(size_t)e * D + hi];
    if (apply_rope) {
      float c, s;
      rope_cs(p, exp(-(2.0 * j / dh) * log_theta), &c, &s);
      float a = x * c - y * s, b = y * c + x * s;
      x = a; y = b;
    }
    store_out<BF16>(out, (size_t)p * D + lo, x);
    store_out<BF16>(out, (size_t)p * D + hi, y);
  }
}

// Window bookkeeping: copy `count` rows and their positions.
// Copy `count` rows and their positions (grid x = row). Copy z of a batched
// launch (grid z) rebases dst and dpos by bd[z] bytes, and src / spos too when
// the source lies in the path's own buffers (src_rebased); a caller source is
// read at src + z * src_stride floats instead.
__global__ void move_rows_kernel(float* dst, int32_t* dpos, const float* __restrict__ src,
                                 const int32_t* __restrict__ spos, int32_t pos_base, int D,
                                 const int64_t* __restrict__ bd, int src_rebased, int64_t src_stride) {
  const int64_t bdel = bd ? bd[blockIdx.z] : 0;
  dst = iskv_rb(dst, bdel);
  dpos = iskv_rb(dpos, bdel);
  if (src_rebased) {
    src = iskv_rb(src, bdel);
    spos = iskv_rb(spos, bdel);
  } else {
    src += (size_t)blockIdx.z * src_stride;
  }
  const int r = blockIdx.x;
  for (int c = threadIdx.x; c < D; c += blockDim.x) dst[(size_t)r * D + c] = src[(size_t)r * D + c];
  if (threadIdx.x == 0 && dpos) dpos[r] = spos ? spos[r] : pos_base + r;
}

__global__ void fill_pos_kernel(int32_t* pos, int count, int32_t v0, int32_t step,
                                const int64_t* __restrict__ bd) {
  pos = iskv_rb(pos, bd ? bd[blockIdx.z] : 0);
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) pos[i] = v0 + step * i;
}

}  // namespace

// Shapes the streaming kernel serves (bf16 output): r_max a multiple of 32
// up to 256, or up to 512 with 256-feature tiles (D a multiple of 256, head_dim
// dividing 256), D a multiple of 128 with whole heads in a 128-feature tile
// (head_dim 32, 64 or 128), and byte offsets of C and of the output within
// the 32-bit range of a buffer descriptor.
static bool recon_wide_tiles(int D, int head_dim) { return D % 256 == 0 && 256 % head_dim == 0; }
bool iskv_recon_stream_ok(const isvd_handle* h, int32_t n_total, int32_t head_dim) {
  const int D = h->cfg.D, R = h->cfg.r_max;
  const size_t cb = (size_t)iskv_coord_bytes(h->cfg);
  const int rmax = recon_wide_tiles(D, head_dim) ? 512 : 256;
  return D % RM_BN == 0 && head_dim % 32 == 0 && RM_BN % head_dim == 0 && R % 32 == 0 && R <= rmax &&
         (size_t)h->n_host * R * cb < ((size_t)1 << 31) && (size_t)n_total * D * 2 < ((size_t)1 << 31);
}

int iskv_launch_reconstruct_batched(const isvd_handle* const* hs, int32_t count, uint16_t* const* outs,
                                    const int32_t* n_totals, const int32_t* ropes, int32_t head_dim,
                                    float rope_theta, hipStream_t s, const float* X_exact,
                                    const int32_t* pos_exact, int32_t n_exact) {
  const isvd_handle* h0 = hs[0];
  const int D = h0->cfg.D, R = h0->cfg.r_max;
  const double lt = log((double)rope_theta);
  RsPaths tab = {};
  int np = 0;
  for (int i = 0; i < count; ++i) {
    if (hs[i]->n_host <= 0) continue;  // nothing compressed: nothing to write
    const isvd_handle* h = hs[i];
    tab.p[np] = RsPath{(const void*)h->C, h->w.Bbf, h->pos, h->w.st, outs[i], h->n_host, n_totals[i],
                       ropes[i] ? 1 : 0, 0};
    ++np;
  }
  if (np > 0) {
    auto go = [&](auto* tag) {
      using TC = std::remove_pointer_t<decltype(tag)>;
      if (recon_wide_tiles(D, head_dim)) {
        // 256-feature tiles (8 waves), one workgroup per CU
        const int T = D / 256;
        const int G = T >= 32 ? 1 : 32 / T;  // 256 workgroups when T divides 32
        const int S = std::max(8 * G, (np + 7) / 8 * 8);  // at least one row group per path
        if (R <= 256)
          hipLaunchKernelGGL((recon_stream_kernel<TC, 8, RS_BM32, 256>), dim3(T * S), dim3(512), 0, s, tab, np, R, R,
                             D, head_dim, lt, T, S);
        else  // 16-row blocks: the ring of staged rows fits beside the wider B operands
          hipLaunchKernelGGL((recon_stream_kernel<TC, 8, 16, 512>), dim3(T * S), dim3(512), 0, s, tab, np, R, R, D,
                             head_dim, lt, T, S);
      } else {
        const int T = D / 128;
        const int G = T >= 64 ? 1 : 64 / T;  // 512 workgroups when T divides 64
        const int S = std::max(8 * G, (np + 7) / 8 * 8);
        hipLaunchKernelGGL((recon_stream_kernel<TC, 4, RS_BM32, 256>), dim3(T * S), dim3(256), 0, s, tab, np, R, R,
                           D, head_dim, lt, T, S);
      }
    };
    if (iskv_bf16_coords(h0->cfg)) go((uint16_t*)nullptr);
    else if (iskv_fp16_coords(h0->cfg)) go((_Float16*)nullptr);
    else go((float*)nullptr);
  }
  if (n_exact > 0)
    hipLaunchKernelGGL(exact_rows_kernel<true>, dim3(n_exact), dim3(256), 0, s, X_exact, pos_exact, D, head_dim,
                       ropes[0], lt, (void*)outs[0], n_totals[0]);
  ISKV_HIP_CHECK(hipGetLastError());
  return ISKV_OK;
}

int iskv_launch_reconstruct(const isvd_handle* h, const float* X_exact, const int32_t* pos_exact,
                            int32_t n_exact, int32_t n_total, int32_t head_dim, int32_t apply_rope,
                            float rope_theta, void* out, int32_t out_dtype, hipStream_t s) {
  const int D = h->cfg.D, R = h->cfg.r_max;
  const int n = h->n_host;
  const double lt = log((double)rope_theta);
  const bool bf = out_dtype == ISKV_OUT_BF16;
  if (n > 0) {
    const int W = (D % 128 == 0 && 128 % head_dim == 0) ? 128 : 64;
    dim3 grid(D / W, (n + 31) / 32);
    const bool mfma = bf && D % RM_BN == 0 && head_dim % 32 == 0 && RM_BN % head_dim == 0 &&
                      R % 8 == 0;
    if (bf && iskv_recon_stream_ok(h, n_total, head_dim)) {
      const int rope = apply_rope ? 1 : 0;
      uint16_t* o = (uint16_t*)out;
      return iskv_launch_reconstruct_batched(&h, 1, &o, &n_total, &rope, head_dim, rope_theta, s, X_exact,
                                             pos_exact, n_exact);
    }
    auto go = [&](auto* Cp) {
      using TC = std::remove_pointer_t<decltype(Cp)>;
      const TC* Cc = Cp;
      if (mfma) {
        const int tiles = D / RM_BN, nrb = (n + RM_BM - 1) / RM_BM;
        const int nwg = (nrb + 7) / 8 * 8 * tiles;
        hipLaunchKernelGGL((recon_mfma_kernel<TC>), dim3(nwg), dim3(256), 0, s, Cc, R, h->w.Bbf, R,
                           h->pos, h->w.st, n, D, head_dim, apply_rope, lt, (uint16_t*)out, n_total,
                           tiles);
      } else if (bf) {
        hipLaunchKernelGGL((recon_kernel<true, TC>), grid, dim3(256), 0, s, Cc, R, h->B, R, h->pos,
                           h->w.st, n, D, head_dim, W, apply_rope, lt, out, n_total);
      } else {
        hipLaunchKernelGGL((recon_kernel<false, TC>), grid, dim3(256), 0, s, Cc, R, h->B, R, h->pos,
                           h->w.st, n, D, head_dim, W, apply_rope, lt, out, n_total);
      }
    };
    if (iskv_bf16_coords(h->cfg)) go((uint16_t*)h->C);
    else if (iskv_fp16_coords(h->cfg)) go((_Float16*)h->C);
    else go(h->C);
  }
  if (n_exact > 0) {
    if (bf)
      hipLaunchKernelGGL(exact_rows_kernel<true>, dim3(n_exact), dim3(256), 0, s, X_exact,
                         pos_exact, D, head_dim, apply_rope, lt, out, n_total);
    else
      hipLaunchKernelGGL(exact_rows_kernel<false>, dim3(n_exact), dim3(256), 0, s, X_exact,
                         pos_exact, D, head_dim, apply_rope, lt, out, n_total);
  }
  ISKV_HIP_CHECK(hipGetLastError());
  return ISKV_OK;
}

int iskv_launch_exact_rows(const float* X_exact, const int32_t* pos_exact, int32_t n_exact, int32_t D,
                           int32_t n_total, int32_t head_dim, int32_t apply_rope, float rope_theta,
                           void* out, int32_t out_dtype, hipStream_t s) {
  if (n_exact <= 0) return ISKV_OK;
  const double lt = log((double)rope_theta);
  if (out_dtype == ISKV_OUT_BF16)
    hipLaunchKernelGGL(exact_rows_kernel<true>, dim3(n_exact), dim3(256), 0, s, X_exact, pos_exact, D,
                       head_dim, apply_rope, lt, out, n_total);
  else
    hipLaunchKernelGGL(exact_rows_kernel<false>, dim3(n_exact), dim3(256), 0, s, X_exact, pos_exact, D,
                       head_dim, apply_rope, lt, out, n_total);
  ISKV_HIP_CHECK(hipGetLastError());
  return ISKV_OK;
}

int iskv_launch_window_move(float* dst_rows, int32_t* dst_pos, const float* src_rows,
                            const int32_t* src_pos, int32_t src_pos_base, int32_t count, int32_t D,
                            hipStream_t s, const int64_t* bd, int32_t bc, int32_t src_rebased,
                            int64_t src_stride) {
  if (count <= 0) return ISKV_OK;
  hipLaunchKernelGGL(move_rows_kernel, bz(dim3(count), bc), dim3(256), 0, s, dst_rows, dst_pos, src_rows,
                     src_pos, src_pos_base, D, bd, src_rebased, src_stride);
  ISKV_HIP_CHECK(hipGetLastError());
  return ISKV_OK;
}

int iskv_launch_fill_pos(int32_t* pos, int32_t count, int32_t value0, int32_t step, hipStream_t s,
                         const int64_t* bd, int32_t bc) {
  if (count <= 0) return ISKV_OK;
  hipLaunchKernelGGL(fill_pos_kernel, bz(dim3((count + 255) / 256), bc), dim3(256), 0, s, pos, count, value0,
                     step, bd);
  ISKV_HIP_CHECK(hipGetLastError());
  return ISKV_OK;
}
