// GQA decode attention with the value history kept factored: the value-side
// decode the iS-KV notes point to (§5.2, §6) that attends with the factors
// instead of rebuilding the dense value cache. For query head h on KV head g,
//   p_h = softmax over every position t of scale * K[t, g] . q_h,
//   o_h = (p_h[pos]^T C) B[g dh : (g + 1) dh, :]^T + p_h[pos_e]^T X_e[:, g dh : (g + 1) dh],
// where C = U diag(sigma) (n x k) and B (D x k) are the value path's factors
// with its rows at positions pos, and X_e the exact value rows. The value
// side reads n k fp32 coordinates instead of n D values.
//
// Split kernel: each workgroup folds rows into running per-head
// (max m, sum l, y = sum_t w_t row_t) for all query heads at once, so each
// row is read once, and writes them as one partial. The first workgroups take
// the compressed rows (y over the k coordinates), the rest the exact rows (y
// over the head's dh-wide slice of X_e); each takes a contiguous share in
// chunks, all in one pass per chunk:
//   scores   wave w scores rows 4 w .. 4 w + 3; lane l holds features
//            16 l .. 16 l + 15 of a key row (KV head l / 8) and the bf16
//            query entries of that head's G query heads; bf16 pair dot
//            products, then a sum over the 8 lanes of the KV head;
//   softmax  thread t updates head t / 8 over rows 4 (t % 8) .. + 3;
//   y        compressed: Y += W C on fp32 matrix cores, wave w owning the
//            coordinate tiles 32 (w + 8 t); exact: wave w owns dims
//            16 w .. 16 w + 15 of every head's slice; the chunk's rows are
//            staged in LDS by direct loads.
// While chunk c is accumulated, chunk c + 1's positions and key rows are in
// flight; its staged rows follow once chunk c has left LDS and land while it
// is scored.
// Merge kernel: per head and 32-column slice, log-sum-exp weights of the
// partials, their weighted sum Y and its share of o = (Y B_g^T + O_e) / L; the
// head's last slice to finish writes o.
#include "iskv_internal.h"

#include <math.h>

#include <type_traits>

namespace {

constexpr int FV_DH = 128;
constexpr int FV_WAVES = 8;                // waves of a split workgroup
constexpr int FV_THREADS = 64 * FV_WAVES;
constexpr int FV_RPW = 4;                  // rows a wave scores per chunk
constexpr int FV_CH = FV_WAVES * FV_RPW;   // compressed rows per chunk
constexpr int FV_CHE = 8;                  // exact rows per chunk (scored by waves 0, 1)
constexpr int FV_EXACT_WG_ROWS = 16;       // exact rows per workgroup, at most
constexpr int FV_HQ = 32;   // largest number of query heads
constexpr int FV_PAD = 4;   // partial record: acc[NA], m, l, 2 unused
constexpr int FV_WP = FV_HQ + 2;  // row pitch of the [row][head] weights (conflict-free reads)

typedef __attribute__((address_space(3))) void* fv_lds_ptr;
typedef __bf16 __attribute__((ext_vector_type(2))) fv_bf2;
typedef float __attribute__((ext_vector_type(16))) fv_f32x16;

__device__ __forceinline__ uint16_t fv_f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// acc + a.lo b.lo + a.hi b.hi on bf16 pairs, in fp32
__device__ __forceinline__ float fv_dot2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(fv_bf2, a), __builtin_bit_cast(fv_bf2, b), acc, false);
}

template <int CTRL>
__device__ __forceinline__ float fv_dpp(float a) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), CTRL, 0xf, 0xf, false));
}
// Sum / maximum over each group of 8 lanes, held by every lane of the group:
// mirror inside the half row (i <-> 7 - i), then swap lane pairs 2 apart and
// 1 apart inside the quad (DPP, no LDS trip).
__device__ __forceinline__ float fv_sum8(float a) {
  a += fv_dpp<0x141>(a);  // row_half_mirror
  a += fv_dpp<0x4e>(a);   // quad_perm [2,3,0,1]
  return a + fv_dpp<0xb1>(a);  // quad_perm [1,0,3,2]
}
__device__ __forceinline__ float fv_max8(float a) {
  a = fmaxf(a, fv_dpp<0x141>(a));
  a = fmaxf(a, fv_dpp<0x4e>(a));
  return fmaxf(a, fv_dpp<0xb1>(a));
}

// Bytes of a staged block of rows x ld elements of esz bytes in LDS, rounded
// up to whole rounds of FV_THREADS lanes x 16 bytes.
__host__ __device__ inline int fv_stage_bytes(int rows, int ld, int esz) {
  return (rows * ld * esz + 16 * FV_THREADS - 1) / (16 * FV_THREADS) * (16 * FV_THREADS);
}

// Dynamic LDS of the split kernel: one compressed chunk (coordinates of esz
// bytes) or one exact block (fp32).
__host__ __device__ inline int fv_split_lds_bytes(int ldc, int esz, int D) {
  const int a = fv_stage_bytes(FV_CH, ldc, esz), b = fv_stage_bytes(FV_CHE, D, 4);
  return a > b ? a : b;
}

// Partial record of one workgroup for one head: [acc[NA], m, l, -, -], with
// NA = 64 KJ for the compressed workgroups (acc over coordinates) and NA = dh
// for the exact ones (acc over the head's slice). Workgroups [0, nwg_c) take
// an even share of the compressed rows each (chunks of FV_CH), the nwg_e
// after them an even share of the exact rows (chunks of FV_CHE).
template <int KJ, int G, typename TC>
__global__ __launch_bounds__(FV_THREADS) void fv_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ K, int n_total, const TC* __restrict__ C,
    int ldc, const int32_t* __restrict__ posc, int nc_rows, int nwg_c, const float* __restrict__ X,
    const int32_t* __restrict__ pose, int ne_rows, int nwg_e, int Hq, int Hkv, float scale,
    float* __restrict__ part_c, float* __restrict__ part_e, int* __restrict__ cnt) {
  constexpr int NA = 64 * KJ, NAE = FV_DH;
  constexpr int NT = NA / (32 * FV_WAVES);  // 32-coordinate MFMA tiles per wave
  const int D = Hkv * FV_DH;
  const int t = threadIdx.x, lane = t & 63;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const bool exact = (int)blockIdx.x >= nwg_c;
  if (blockIdx.x == 0 && t < Hq) cnt[t] = 0;  // merge arrival counters of this call
  // block geometry: rows R (ld), positions, rows per chunk, and this
  // workgroup's even share [r_begin, r_end) of the rows
  const char* const R = exact ? (const char*)X : (const char*)C;
  const int ld = exact ? D : ldc;
  const int esz = exact ? 4 : (int)sizeof(TC);  // bytes per staged element
  const int32_t* const pos = exact ? pose : posc;
  const int nrows = exact ? ne_rows : nc_rows;
  const int rpc = exact ? FV_CHE : FV_CH;
  const int wid = exact ? (int)blockIdx.x - nwg_c : (int)blockIdx.x;
  const int nwg = exact ? nwg_e : nwg_c;
  const int r_begin = (int)(((int64_t)wid * nrows) / nwg);
  const int r_end = (int)(((int64_t)(wid + 1) * nrows) / nwg);
  const int nchunk = (r_end - r_begin + rpc - 1) / rpc;

  __shared__ float S[FV_HQ * FV_CH + 64];  // logits [head][row]; 64 spare slots
  __shared__ float scs[FV_HQ];             // per-head rescale of this chunk
  __shared__ float W2[FV_CH * FV_WP];      // weights [row][head]
  extern __shared__ float4 fv_stage[];
  float* const buf = (float*)fv_stage;  // exact rows (fp32)
  const TC* const bufc = (const TC*)fv_stage;  // compressed rows (stored coordinates)
  const int sbytes = fv_stage_bytes(rpc, ld, esz);

  // query entries of this lane's 16 features for the G heads of its KV head
  const int gq = lane >> 3, sub = lane & 7;
  const bool fl = gq < Hkv;
  const int foff = fl ? 16 * lane : 0;
  uint32_t qp[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const int h = min(gq * G + hh, Hq - 1);
    const uint4* src = (const uint4*)(q + (size_t)h * FV_DH + 16 * sub);
    const uint4 a = src[0], b = src[1];
    qp[hh][0] = a.x; qp[hh][1] = a.y; qp[hh][2] = a.z; qp[hh][3] = a.w;
    qp[hh][4] = b.x; qp[hh][5] = b.y; qp[hh][6] = b.z; qp[hh][7] = b.w;
  }
  // compressed: y = W C on fp32 MFMA 32x32x2, wave w owning the coordinate
  // tiles 32 (w + 8 tt) .. + 31; lane l holds acc[tt][v] for head
  // 8 (v / 4) + 4 (l / 32) + v % 4 and coordinate 32 (w + 8 tt) + l % 32
  const int kk = lane >> 5, mi = lane & 31;
  fv_f32x16 accm[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
#pragma unroll
    for (int v = 0; v < 16; ++v) accm[tt][v] = 0.f;
  // exact: lane l holds heads 4 hg .. 4 hg + 3, dims 16 wave + 2 cg + e of
  // each head's slice
  const int hg = lane >> 3, cg = lane & 7;
  float acce[4][2] = {{0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}, {0.f, 0.f}};
  float m_h = -INFINITY, l_h = 0.f;  // head t / 8 (softmax threads t < 256)

  // rows [r0, r0 + rpc) of chunk c into LDS; they are contiguous in memory
  // and bytes past row r_end read as zero through the buffer descriptor
  auto stage = [&](int c) {
    const int r0 = r_begin + c * rpc;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(R + (size_t)r0 * ld * esz), 0, min(rpc, r_end - r0) * ld * esz, 0x00020000);
    const int nd = sbytes / (16 * FV_THREADS);
    for (int v = 0; v < nd; ++v) {
      const int base = 1024 * (FV_WAVES * v + wv);  // bytes
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (fv_lds_ptr)((char*)fv_stage + base), 16, base + 16 * lane, 0, 0,
                                               0);
    }
  };
  // positions of this wave's rows (uniform: scalar loads)
  auto load_pos = [&](int c, int (&pr)[FV_RPW]) {
#pragma unroll
    for (int rho = 0; rho < FV_RPW; ++rho) pr[rho] = pos[min(r_begin + c * rpc + FV_RPW * wv + rho, r_end - 1)];
  };
  auto row_ok = [&](int c, int rho, int p) {
    return FV_RPW * wv + rho < rpc && r_begin + c * rpc + FV_RPW * wv + rho < r_end && p >= 0 && p < n_total;
  };
  auto load_k = [&](int c, const int (&pr)[FV_RPW], uint4 (&kv)[FV_RPW][2]) {
#pragma unroll
    for (int rho = 0; rho < FV_RPW; ++rho) {
      const int pl = row_ok(c, rho, pr[rho]) ? pr[rho] : 0;
      const uint4* src = (const uint4*)(K + (size_t)pl * D + foff);
      kv[rho][0] = src[0];
      kv[rho][1] = src[1];
    }
  };
  int pr[FV_RPW];
  uint4 kv[FV_RPW][2];
  if (nchunk > 0) {
    stage(0);
    load_pos(0, pr);
    load_k(0, pr, kv);
  }
  for (int c = 0; c < nchunk; ++c) {
    const bool has_next = c + 1 < nchunk;
    int prn[FV_RPW];
    if (has_next) load_pos(c + 1, prn);
    // ---- scores of rows FV_RPW wave + rho: lanes of KV head gq with sub < G
    // store head gq G + sub
#pragma unroll
    for (int rho = 0; rho < FV_RPW; ++rho) {
      float v = -INFINITY;
      if (row_ok(c, rho, pr[rho])) {
        const uint32_t kw[8] = {kv[rho][0].x, kv[rho][0].y, kv[rho][0].z, kv[rho][0].w,
                                kv[rho][1].x, kv[rho][1].y, kv[rho][1].z, kv[rho][1].w};
        float a[G];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          float s0 = 0.f, s1 = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s0 = fv_dot2(qp[hh][e], kw[e], s0);
            s1 = fv_dot2(qp[hh][4 + e], kw[4 + e], s1);
          }
          a[hh] = fv_sum8(s0 + s1);
        }
        v = a[0];
#pragma unroll
        for (int hh = 1; hh < G; ++hh) v = (sub == hh) ? a[hh] : v;
        v *= scale;
      }
      const bool mine = fl && sub < G && gq * G + sub < Hq;
      S[mine ? (gq * G + sub) * FV_CH + FV_RPW * wv + rho : FV_HQ * FV_CH + lane] = v;
    }
    // every wave's staged rows of chunk c have landed before the barrier
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // ---- softmax update of head t / 8 over rows 4 (t % 8) .. + 3 by the
    // first 256 threads (heads past Hq hold unused values; rows past the
    // block hold -inf)
    if (t < 8 * FV_HQ) {
      const float4 s4 = *(const float4*)&S[(t >> 3) * FV_CH + 4 * (t & 7)];
      const float mx = fv_max8(fmaxf(fmaxf(s4.x, s4.y), fmaxf(s4.z, s4.w)));
      const float mn = fmaxf(m_h, mx);
      const float sc = (mn == -INFINITY) ? 1.f : __expf(m_h - mn);
      auto ex = [&](float s) { return (s == -INFINITY) ? 0.f : __expf(s - mn); };
      const float4 w4 = {ex(s4.x), ex(s4.y), ex(s4.z), ex(s4.w)};
      l_h = l_h * sc + fv_sum8((w4.x + w4.y) + (w4.z + w4.w));
      m_h = mn;
      float* const wp = &W2[4 * (t & 7) * FV_WP + (t >> 3)];
      wp[0] = w4.x;
      wp[FV_WP] = w4.y;
      wp[2 * FV_WP] = w4.z;
      wp[3 * FV_WP] = w4.w;
      if ((t & 7) == 0) scs[t >> 3] = sc;
    }
    __syncthreads();
    // ---- next chunk's key rows in flight while this one is accumulated
    if (has_next) {
#pragma unroll
      for (int rho = 0; rho < FV_RPW; ++rho) pr[rho] = prn[rho];
      load_k(c + 1, pr, kv);
    }
    // ---- accumulate: y_h = sc_h y_h + sum_rho w[h][rho] row_rho over the
    // chunk's valid rows
    const int vr = min(rpc, r_end - (r_begin + c * rpc));
    if (exact) {
      const float4 sc4 = *(const float4*)&scs[4 * hg];
      const float sc[4] = {sc4.x, sc4.y, sc4.z, sc4.w};
      // the KV head of query head 4 hg + hh and this lane's dims in its slice
      int col[4];
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        col[hh] = (min(4 * hg + hh, Hq - 1) / G) * FV_DH + 16 * wv + 2 * cg;
        acce[hh][0] *= sc[hh];
        acce[hh][1] *= sc[hh];
      }
      for (int r = 0; r < vr; ++r) {
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) {
          const float w = W2[r * FV_WP + 4 * hg + hh];
          const float2 x = *(const float2*)(buf + r * ld + col[hh]);
          acce[hh][0] = fmaf(w, x.x, acce[hh][0]);
          acce[hh][1] = fmaf(w, x.y, acce[hh][1]);
        }
      }
    } else {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 sc4 = *(const float4*)&scs[8 * q4 + 4 * kk];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          accm[tt][4 * q4] *= sc4.x;
          accm[tt][4 * q4 + 1] *= sc4.y;
          accm[tt][4 * q4 + 2] *= sc4.z;
          accm[tt][4 * q4 + 3] *= sc4.w;
        }
      }
      // k-step s pairs row s (lanes < 32) with row 16 + s (lanes >= 32):
      // A = w[head mi][16 kk + s], B = row 16 kk + s at coordinate n
      const float* wcol = &W2[16 * kk * FV_WP + mi];
      int nb[NT];  // coordinate column of each tile in the staged rows (clamped) and its mask
      bool nok[NT];
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        const int n = 32 * (wv + FV_WAVES * tt) + mi;
        nok[tt] = n < ld;
        nb[tt] = min(n, ld - 1);
      }
      const TC* const brow0 = bufc + 16 * kk * ld;
      if (vr >= 16) {
        // operands of all 16 k-steps first, then the MFMA chain
        float av[16], bv[16][NT];
#pragma unroll
        for (int st = 0; st < 16; ++st) {
          av[st] = wcol[st * FV_WP];
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) bv[st][tt] = iskv_ld(brow0 + st * ld + nb[tt]);
        }
#pragma unroll
        for (int st = 0; st < 16; ++st)
#pragma unroll
          for (int tt = 0; tt < NT; ++tt)
            accm[tt] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[st], nok[tt] ? bv[st][tt] : 0.f, accm[tt], 0, 0, 0);
      } else {
        for (int st = 0; st < vr; ++st) {
          const float a = wcol[st * FV_WP];
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) {
            const float b = iskv_ld(brow0 + st * ld + nb[tt]);
            accm[tt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, nok[tt] ? b : 0.f, accm[tt], 0, 0, 0);
          }
        }
      }
    }
    __syncthreads();
    // the next chunk's rows land in LDS while it is scored
    if (has_next) stage(c + 1);
  }
  // partial records of this workgroup
  const int rec = exact ? NAE + FV_PAD : NA + FV_PAD;
  float* const pbase = (exact ? part_e : part_c) + (size_t)wid * Hq * rec;
  const int na = exact ? NAE : NA;
  if (t < 8 * FV_HQ && (t >> 3) < Hq && (t & 7) == 0) {
    float* dst = pbase + (size_t)(t >> 3) * rec + na;
    dst[0] = m_h;
    dst[1] = l_h;
  }
  if (exact) {
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      const int h = 4 * hg + hh;
      if (h < Hq) *(float2*)(pbase + (size_t)h * rec + 16 * wv + 2 * cg) = float2{acce[hh][0], acce[hh][1]};
    }
  } else {
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int h = 8 * (v >> 2) + 4 * kk + (v & 3);
        if (h < Hq) pbase[(size_t)h * rec + 32 * (wv + FV_WAVES * tt) + mi] = accm[tt][v];
      }
  }
}

// Merge of the partials of head h = blockIdx.x over columns 32 y .. 32 y + 31,
// and that slice's share of the output. y < NC / 32 takes the compressed
// partials (nc, width NC = 64 KJ), the next dh / 32 the exact ones (ne, width
// dh). Each workgroup forms the head's maximum M and sum
// L = sum_s exp(m_s - M) l_s itself, then
//   Y[j] = sum_s exp(m_s - M) acc_s[j]       (j in the slice)
//   opart[h][y][d] = sum_j Y[j] B[g dh + d][j]  (compressed, j < k) or Y[d] (exact dims)
// Thread t sums partials t / 8 + 32 i over columns 4 (t % 8) .. + 3; the
// first FV_MPF of them, and its B entries, are loaded before the weights are
// known. The last workgroup of head h to finish (counted in cnt[h], zeroed
// by the split kernel) sums opart[h][.][d] in slice order and writes
// o[h][d] = sum / L as bf16.
constexpr int FV_MPF = 8;
template <int KJ, int G>
__global__ __launch_bounds__(256) void fv_merge_kernel(const float* __restrict__ pc, int nc,
                                                       const float* __restrict__ pe, int ne, int Hq,
                                                       const float* __restrict__ Bv, int ldb,
                                                       const int32_t* __restrict__ st, float* __restrict__ opart,
                                                       int* __restrict__ cnt, uint16_t* __restrict__ out) {
  constexpr int NC = 64 * KJ, RC = NC + FV_PAD, RE = FV_DH + FV_PAD, NSL = (NC + FV_DH) / 32;
  const int h = blockIdx.x, sl = blockIdx.y, g = h / G;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int kval = st[ST_K];
  __shared__ float redm[4], redl[4];
  __shared__ float4 red[32][8];
  __shared__ float Ys[32];
  __shared__ int last;
  extern __shared__ float ms[];  // [2 (nc + ne)]: m_s (then weights), l_s
  float* const ls = ms + nc + ne;
  const bool ex = sl >= NC / 32;
  const int c0 = 32 * (ex ? sl - NC / 32 : sl);
  const float* src = (ex ? pe + (size_t)h * RE : pc + (size_t)h * RC) + c0 + 4 * (t & 7);
  const size_t stride = (size_t)Hq * (ex ? RE : RC);
  const int n = ex ? ne : nc;
  float4 v[FV_MPF];  // partials past n: row n - 1 again, weighted 0
  if (n > 0) {
#pragma unroll
    for (int i = 0; i < FV_MPF; ++i) v[i] = *(const float4*)(src + (size_t)min((t >> 3) + 32 * i, n - 1) * stride);
  }
  // B[g dh + t / 2][c0 + 16 (t % 2) + 4 i .. + 3] (columns past the row clamped, masked below)
  float4 bq[4];
  if (!ex) {
    const float* brow = Bv + (size_t)(g * FV_DH + (t >> 1)) * ldb;
#pragma unroll
    for (int i = 0; i < 4; ++i) bq[i] = *(const float4*)(brow + min(c0 + 16 * (t & 1) + 4 * i, ldb - 4));
  }
  float m = -INFINITY;
  for (int s = t; s < nc + ne; s += 256) {
    const float* r = (s < nc) ? pc + ((size_t)s * Hq + h) * RC + NC : pe + ((size_t)(s - nc) * Hq + h) * RE + FV_DH;
    const float2 ml = *(const float2*)r;
    ms[s] = ml.x;
    ls[s] = ml.y;
    m = fmaxf(m, ml.x);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if (lane == 0) redm[wave] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(redm[0], redm[1]), fmaxf(redm[2], redm[3]));
  float l = 0.f;
  for (int s = t; s < nc + ne; s += 256) {
    const float w = (ms[s] == -INFINITY) ? 0.f : __expf(ms[s] - M);
    l += w * ls[s];
    ms[s] = w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
  if (lane == 0) redl[wave] = l;
  __syncthreads();
  const float* w0 = ms + (ex ? nc : 0);
  float4 y = {0.f, 0.f, 0.f, 0.f};
  auto add = [&](float w, float4 x) {
    y.x = fmaf(w, x.x, y.x);
    y.y = fmaf(w, x.y, y.y);
    y.z = fmaf(w, x.z, y.z);
    y.w = fmaf(w, x.w, y.w);
  };
#pragma unroll
  for (int i = 0; i < FV_MPF; ++i) {
    const int s = (t >> 3) + 32 * i;
    if (s < n) add(w0[s], v[i]);
  }
  for (int s = (t >> 3) + 32 * FV_MPF; s < n; s += 32) add(w0[s], *(const float4*)(src + (size_t)s * stride));
  red[t >> 3][t & 7] = y;
  __syncthreads();
  if (t < 32) {
    float sum = 0.f;
#pragma unroll 8
    for (int q = 0; q < 32; ++q) sum += ((const float*)red[q])[t];
    Ys[t] = (ex || c0 + t < kval) ? sum : 0.f;
  }
  __syncthreads();
  // opart goes through agent-coherent stores and loads (no cache-wide fences):
  // this workgroup's stores have completed before its count is added, and the
  // last workgroup reads them after seeing the final count
  float* const op = opart + ((size_t)h * NSL + sl) * FV_DH;
  if (ex) {
    if (t < FV_DH)
      __hip_atomic_store(op + t, (t >= c0 && t < c0 + 32) ? Ys[t - c0] : 0.f, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  } else {
    float o = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 16 * (t & 1) + 4 * i;  // column within the slice
      const float bb[4] = {bq[i].x, bq[i].y, bq[i].z, bq[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) o = fmaf(Ys[j + e], (c0 + j + e < kval) ? bb[e] : 0.f, o);
    }
    o += fv_dpp<0xb1>(o);  // the two threads of row t / 2
    if ((t & 1) == 0) __hip_atomic_store(op + (t >> 1), o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (t == 0) last = __hip_atomic_fetch_add(&cnt[h], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == NSL - 1;
  __syncthreads();
  if (last) {
    if (t < FV_DH) {
      const float* oh = opart + (size_t)h * NSL * FV_DH + t;
      float o = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < NSL; ++s2) o += __hip_atomic_load(oh + s2 * FV_DH, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      out[(size_t)h * FV_DH + t] = fv_f2bf(o / (redl[0] + redl[1] + redl[2] + redl[3]));
    }
  }
}

// Compute units of the current device (one split workgroup of 8 waves
// fills one).
inline int fv_cu_count() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}
inline int fv_nwg_e(int rows) { return (rows + FV_EXACT_WG_ROWS - 1) / FV_EXACT_WG_ROWS; }
// Compressed workgroups: the CUs left beside the exact ones, each taking an
// even share of the rows.
inline int fv_nwg_c(int rows, int exact_rows) {
  const int c = (rows + FV_CH - 1) / FV_CH;
  const int room = fv_cu_count() - fv_nwg_e(exact_rows);
  const int cap = room > 64 ? room : 64;
  return c < cap ? c : cap;
}
inline int fv_kj(int r_max) { return r_max <= 256 ? 4 : 8; }

// Raise a kernel's dynamic LDS limit once per kernel (above 64 KB it must be
// asked for explicitly).
template <typename F>
hipError_t fv_lds_limit(F* fn, size_t bytes) {
  static size_t set = 0;
  if (bytes <= set) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) set = bytes;
  return e;
}

}  // namespace

size_t iskv_attend_fv_ws_bytes(int32_t n_c, int32_t n_exact, int32_t Hq, int32_t r_max) {
  const size_t nc = (size_t)fv_nwg_c(n_c, n_exact), ne = (size_t)fv_nwg_e(n_exact);
  const size_t NC = 64 * fv_kj(r_max), NSL = (NC + FV_DH) / 32;
  return (nc * Hq * (NC + FV_PAD) + ne * Hq * (FV_DH + FV_PAD) + (size_t)Hq * NSL * FV_DH + (size_t)Hq) *
         sizeof(float);
}

int iskv_launch_attend_fv(const uint16_t* q, const uint16_t* K, const isvd_handle* hv, const float* X_exact,
                          const int32_t* pos_exact, int32_t n_exact, int32_t n_total, int32_t Hq, int32_t Hkv,
                          float scale, uint16_t* out, void* ws, size_t ws_bytes, hipStream_t s) {
  const int n_c = hv->n_host, R = hv->cfg.r_max, D = hv->cfg.D;
  const int kj = fv_kj(R), NC = 64 * kj, NSL = (NC + FV_DH) / 32;
  if (ws_bytes < iskv_attend_fv_ws_bytes(n_c, n_exact, Hq, R)) return ISKV_EWORKSPACE;
  const int nc = fv_nwg_c(n_c, n_exact), ne = fv_nwg_e(n_exact);
  float* pc = (float*)ws;
  float* pe = pc + (size_t)nc * Hq * (NC + FV_PAD);
  float* opart = pe + (size_t)ne * Hq * (FV_DH + FV_PAD);
  int* cnt = (int*)(opart + (size_t)Hq * NSL * FV_DH);
  const int G = Hq / Hkv;
  const size_t lds = (size_t)fv_split_lds_bytes(R, iskv_coord_bytes(hv->cfg), D);
  auto launch = [&](auto kj_c, auto g_c) -> hipError_t {
    constexpr int KJ = decltype(kj_c)::value, GG = decltype(g_c)::value;
    auto split = [&](auto* Cp) -> hipError_t {
      using TC = std::remove_pointer_t<decltype(Cp)>;
      const hipError_t e = fv_lds_limit(fv_split_kernel<KJ, GG, TC>, lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((fv_split_kernel<KJ, GG, TC>), dim3(nc + ne), dim3(FV_THREADS), lds, s, q, K, n_total,
                         (const TC*)Cp, R, hv->pos, n_c, nc, X_exact, pos_exact, n_exact, ne, Hq, Hkv, scale, pc, pe,
                         cnt);
      return hipSuccess;
    };
    const hipError_t e = iskv_bf16_coords(hv->cfg)   ? split((uint16_t*)hv->C)
                         : iskv_fp16_coords(hv->cfg) ? split((_Float16*)hv->C)
                                                     : split(hv->C);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((fv_merge_kernel<KJ, GG>), dim3(Hq, NSL), dim3(256), (size_t)2 * (nc + ne) * sizeof(float), s,
                       pc, nc, pe, ne, Hq, hv->B, R, hv->w.st, opart, cnt, out);
    return hipGetLastError();
  };
  auto by_g = [&](auto kj_c) -> hipError_t {
    if (G == 1) return launch(kj_c, std::integral_constant<int, 1>{});
    if (G == 2) return launch(kj_c, std::integral_constant<int, 2>{});
    return launch(kj_c, std::integral_constant<int, 4>{});
  };
  ISKV_HIP_CHECK(kj == 4 ? by_g(std::integral_constant<int, 4>{}) : by_g(std::integral_constant<int, 8>{}));
  return ISKV_OK;
}
