// Device code of the batched path (1 < batch <= 32): per-sequence predictor
// masks, their union, and the FFN over the union's rows as gathered dense
// GEMMs on the matrix cores (v_mfma_f32_32x32x16_f16).
//
// Every GEMM has the batch as its M dimension (padded to 32 with zero rows)
// and a weight matrix whose rows are contiguous along K:
//   t  = X A^T     (K = d)      k_bpred1 -> per-split partials, k_bsplit_t
//   s  = T B^T + c (K = r)      k_bscore: masks [ffn][32] and the union
//   z  = X W^T     (K = d)      k_bup: gathered up/gate rows of the union
//   y  = H Wd      (K = union)  k_bdown: W_downT rows staged through LDS
// The activations (x, t, h) are split into fp16 hi + lo parts (x = hi + lo to
// about 22 bits), and every product is run twice (hi, lo) with fp32
// accumulation; fp16 and Q4_0 weights are exact in fp16 (Q4_0 as q - 8, its
// scale applied in fp32).  So the matrix cores give fp32-level results: the
// predictor's scores stay within the threshold band of the single-token path
// and the FFN within the same tolerance.  Each activation row b is scaled by
// a power of two s_b before the split, so that its largest magnitude lies in
// [2^13, 2^14): no value overflows fp16 (65504) and small rows keep their lo
// bits out of the fp16 subnormals.  A product's row b is then s_b times the
// true one, and the consumer multiplies it by 1 / s_b, exactly.
//
// MFMA 32x32x16 f16 operand layout (lane l, e = 0..7): A[row l%32][k = 8*(l/32)
// + e], B[k = 8*(l/32) + e][col l%32]; accumulator element 4g+v of lane l is
// D[row 8g + 4*(l/32) + v][col l%32].
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pi_kernels.hpp"

namespace pib {

using namespace pik;

constexpr int BM = 32;   // batch rows of every GEMM (padded)

typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f16v mfma(h8v a, h8v b, f16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// A operands ([32][K] fp16: x, t and h, K a multiple of 16) are stored in
// operand order: the 32 x 16 block of K step s is 512 contiguous halves, lane
// l's 8 values (row l % 32, k = 16 s + 8 (l / 32) + e) at 8 l.  A wave then
// reads one K step as 1 KB of contiguous memory instead of 32 rows x 32 B.
__host__ __device__ constexpr size_t aop(int row, int k) {
  return (size_t)(k >> 4) * 512 + (size_t)((k >> 3) & 1) * 256 + (size_t)row * 8 + (k & 7);
}

// The power of two s with m s in [2^13, 2^14) for a row of largest magnitude
// m (1 for a zero or non-finite m).
__device__ __forceinline__ float pow2_scale(float m) {
  if (!(m > 0.f) || !__builtin_isfinite(m)) return 1.f;
  int e;
  (void)frexpf(m, &e);                     // m = f 2^e, f in [0.5, 1)
  return ldexpf(1.f, min(max(14 - e, -120), 120));
}

// fp32 value -> (hi, lo) fp16 pair with hi + lo ~ v to about 22 bits
__device__ __forceinline__ void split_f16(float v, _Float16* hi, _Float16* lo) {
  const _Float16 h = (_Float16)v;
  *hi = h;
  *lo = (_Float16)(v - (float)h);
}

// 8 fp16 (16 bytes) of an fp16 matrix as an MFMA operand
__device__ __forceinline__ h8v as_h8(uint4 c) { return __builtin_bit_cast(h8v, c); }

typedef _Float16 h2v __attribute__((ext_vector_type(2)));

// 8 weights of a Q4_0 block as (q - 8) in fp16, exact: nibbles of 8 of its
// bytes (the words w0, w1), low (hi_nib = false) or high nibble.  Two bytes at a
// time go to the low bits of two 16-bit lanes (a byte permute), the nibble is
// masked into the mantissa of the fp16 1024 (0x6400 | q = 1024 + q), and 1032 is
// subtracted from both lanes at once: four operations per pair of weights.
__device__ __forceinline__ h8v q4_h8w(uint32_t w0, uint32_t w1, bool hi_nib) {
  const uint32_t wd[2] = {w0, w1};
  const h2v off = {(_Float16)1032.f, (_Float16)1032.f};
  h8v r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // bytes 2 (k % 2) and 2 (k % 2) + 1 of word k / 2 into the low bytes of two 16-bit lanes
    uint32_t p = __builtin_amdgcn_perm(0u, wd[k >> 1], (k & 1) ? 0x0c030c02u : 0x0c010c00u);
    if (hi_nib) p >>= 4;
    const uint32_t v = (p & 0x000F000Fu) | 0x64006400u;
    const h2v h = __builtin_bit_cast(h2v, v) - off;
    r[2 * k] = h[0];
    r[2 * k + 1] = h[1];
  }
  return r;
}

// A row's Q4_0 blocks 2m and 2m + 1 for an MFMA operand whose lane half h
// (lanes 32 h .. 32 h + 31, one row per lane) needs bytes [8 h, 8 h + 8) of
// each: half h loads block 2m + h whole, and two swaps of the halves' words
// (v_permlane32_swap exchanges a register's upper 32 lanes with another's
// lower 32) leave each half its bytes of block 2m in lo and of 2m + 1 in hi.
__device__ __forceinline__ void q4_pair(uint4 c, uint2& lo, uint2& hi) {
  const auto a = __builtin_amdgcn_permlane32_swap(c.x, c.z, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(c.y, c.w, false, false);
  lo = make_uint2(a[0], b[0]);
  hi = make_uint2(a[1], b[1]);
}

// ------------------------------------------------------------------- glue
// One block per padded sequence row b < 32.  Rows b < B: x' = glue(x_prev[b],
// sum of np partials y[p][b]) (np = 0: x' = x_prev[b]); x' goes to x_out[b]
// (and x_trace[b]) in fp32 and, times its row scale sx[b], to xh/xl row b
// (operand order) as fp16 hi/lo.  Rows b >= B are written as zeros in xh/xl
// so that they contribute nothing to any product.  Block b also clears the
// row maximum hmax[b] of the layer's h.
constexpr int BG_T = 1024;               // threads of a glue block
// BG_V float4 per thread held at once (d <= 4096 BG_V); the partial vectors are
// read 16 / BG_V at a time, so at the usual widths all of them are in flight
// together with x (bd_splits(d) <= 16 / BG_V + 1)
template <int BG_V>
__global__ void __launch_bounds__(BG_T)
k_bglue(const float* __restrict__ x_prev, const float* __restrict__ y_part, int np, int B, int d,
        float* __restrict__ x_out, float* __restrict__ x_trace, _Float16* __restrict__ xh,
        _Float16* __restrict__ xl, float* __restrict__ sx, uint32_t* __restrict__ hmax) {
  __shared__ float red[BG_T / WAVE];
  __shared__ float mred[BG_T / WAVE];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int nv = d / 4;
  if (tid == 0) hmax[b] = 0u;
  if (b >= B) {
    if (tid == 0) sx[b] = 1.f;
    for (int k = tid; k < d; k += blockDim.x) {
      xh[aop(b, k)] = (_Float16)0.f;
      xl[aop(b, k)] = (_Float16)0.f;
    }
    return;
  }
  const size_t ystride = (size_t)BM * d;   // partial p of row b is at y_part + p*32*d + b*d
  const float4* x4 = reinterpret_cast<const float4*>(x_prev + (size_t)b * d);
  // this thread's float4 elements k = tid + BG_T j; every load is issued before
  // the first add (indices past the row read its last vector and are dropped)
  float4 v[BG_V];
#pragma unroll
  for (int j = 0; j < BG_V; ++j) v[j] = x4[min(tid + BG_T * j, nv - 1)];
  if (np > 0) {
    float4 y[BG_V];
#pragma unroll
    for (int j = 0; j < BG_V; ++j)
      y[j] = reinterpret_cast<const float4*>(y_part + (size_t)b * d)[min(tid + BG_T * j, nv - 1)];
    // the other partials, GP at a time: all their loads before the first add,
    // added in partial order (partials past np are read clamped and dropped)
    constexpr int GP = 16 / BG_V;
    for (int p0 = 1; p0 < np; p0 += GP) {
      float4 u[GP][BG_V];
#pragma unroll
      for (int g = 0; g < GP; ++g)
#pragma unroll
        for (int j = 0; j < BG_V; ++j)
          u[g][j] = reinterpret_cast<const float4*>(y_part + min(p0 + g, np - 1) * ystride +
                                                    (size_t)b * d)[min(tid + BG_T * j, nv - 1)];
#pragma unroll
      for (int g = 0; g < GP; ++g)
#pragma unroll
        for (int j = 0; j < BG_V; ++j) {
          const bool on = p0 + g < np;
          y[j].x += on ? u[g][j].x : 0.f;
          y[j].y += on ? u[g][j].y : 0.f;
          y[j].z += on ? u[g][j].z : 0.f;
          y[j].w += on ? u[g][j].w : 0.f;
        }
    }
#pragma unroll
    for (int j = 0; j < BG_V; ++j) {
      v[j].x += y[j].x;
      v[j].y += y[j].y;
      v[j].z += y[j].z;
      v[j].w += y[j].w;
    }
  }
  float inv = 1.f;
  if (np > 0) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < BG_V; ++j) {
      if (tid + BG_T * j < nv) {
        ss = fmaf(v[j].x, v[j].x, ss);
        ss = fmaf(v[j].y, v[j].y, ss);
        ss = fmaf(v[j].z, v[j].z, ss);
        ss = fmaf(v[j].w, v[j].w, ss);
      }
    }
    ss = wave_sum(ss);
    if (lane == 0) red[w] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < BG_T / WAVE; ++i) tot += red[i];
    inv = 1.0f / sqrtf(tot / (float)d + 1e-6f);
  }
  // the row's largest |x'| and its scale
  float mx = 0.f;
#pragma unroll
  for (int j = 0; j < BG_V; ++j)
    if (tid + BG_T * j < nv)
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[j].x * inv), fabsf(v[j].y * inv)), fmaxf(fabsf(v[j].z * inv), fabsf(v[j].w * inv))));
  mx = wave_max(mx);
  if (lane == 0) mred[w] = mx;
  __syncthreads();
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < BG_T / WAVE; ++i) m = fmaxf(m, mred[i]);
  const float sc = pow2_scale(m);
  if (tid == 0) sx[b] = sc;
#pragma unroll
  for (int j = 0; j < BG_V; ++j) {
    const int k4 = tid + BG_T * j;
    if (k4 >= nv) continue;
    const float o[4] = {v[j].x * inv, v[j].y * inv, v[j].z * inv, v[j].w * inv};
    if (x_out) reinterpret_cast<float4*>(x_out + (size_t)b * d)[k4] = make_float4(o[0], o[1], o[2], o[3]);
    if (x_trace) reinterpret_cast<float4*>(x_trace + (size_t)b * d)[k4] = make_float4(o[0], o[1], o[2], o[3]);
    _Float16 hh[4], ll[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split_f16(o[e] * sc, &hh[e], &ll[e]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xh[aop(b, 4 * k4 + e)] = hh[e];
      xl[aop(b, 4 * k4 + e)] = ll[e];
    }
  }
}

// ------------------------------------------------------------ predictor 1
// Partial t over one K split: t_part[ks][b][j] = sum_{k in split ks} x[b][k] A[j][k].
// Block (jt, ks): 32 rows of A (j = 32 jt + col); the split's K range is dealt
// to the 4 waves in 16-wide steps, KU steps per batch of loads; wave partials
// are summed through LDS in a fixed order.
constexpr int KU = 8;    // K steps (of 16) per batch of loads in the MFMA loops

// hi/lo operand pair of 8 fp32 weights
__device__ __forceinline__ void split8(const float* __restrict__ p, h8v* hi, h8v* lo) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    _Float16 h, l;
    split_f16(v[e], &h, &l);
    (*hi)[e] = h;
    (*lo)[e] = l;
  }
}

// acc += X[rows of this lane][K window] * W[row][K window] over KU steps of 16,
// starting at k; X given as hi/lo fp16 [32][K] in operand order, W rows
// contiguous along K.
// All loads of the window are issued before the first MFMA, with no branch
// among them: steps at or past kend load a clamped address and multiply a
// zero X operand instead.
template <int WT>
__device__ __forceinline__ void mfma_window(f16v& acc, const _Float16* __restrict__ xh,
                                            const _Float16* __restrict__ xl, const void* __restrict__ W,
                                            size_t row, size_t ldw, int k, int kend, int kstride, int lane) {
  const int half = lane / 32;
  h8v ah[KU], al[KU], bw[KU], bl[KU];
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const int ks = min(k + u * kstride, kend - 16), kk = ks + 8 * half;
    const size_t xo = (size_t)(ks >> 4) * 512 + 8 * lane;
    ah[u] = *reinterpret_cast<const h8v*>(xh + xo);
    al[u] = *reinterpret_cast<const h8v*>(xl + xo);
    if constexpr (WT == DT_F16) {
      bw[u] = as_h8(*reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W) + row * ldw + kk));
    } else {
      split8(static_cast<const float*>(W) + row * ldw + kk, &bw[u], &bl[u]);
    }
  }
  PI_ISSUE_FENCE();
  const h8v z8 = {};
#pragma unroll
  for (int u = 0; u < KU; ++u) {
    const bool ok = k + u * kstride < kend;
    const h8v a = ok ? ah[u] : z8, b = ok ? al[u] : z8;
    acc = mfma(a, bw[u], acc);
    acc = mfma(b, bw[u], acc);
    if constexpr (WT == DT_F32) acc = mfma(a, bl[u], acc);
  }
}

template <int PT>
__global__ void __launch_bounds__(256)
k_bpred1(const void* __restrict__ A, int r, int d, int ksplit, const _Float16* __restrict__ xh,
         const _Float16* __restrict__ xl, float* __restrict__ t_part) {
  __shared__ float red[4][BM * BM];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int njt = (r + BM - 1) / BM;
  const int jt = blockIdx.x % njt, ks = blockIdx.x / njt;
  const int col = lane % 32, half = lane / 32;
  const int j = min(jt * BM + col, r - 1);
  const int kper = ((d + ksplit - 1) / ksplit + 15) / 16 * 16;
  const int k0 = ks * kper, k1 = min(d, k0 + kper);
  f16v acc = {};
  for (int k = k0 + 16 * w; k < k1; k += 4 * 16 * KU)
    mfma_window<PT>(acc, xh, xl, A, (size_t)j, d, k, k1, 4 * 16, lane);
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[w][(8 * g + 4 * half + v) * BM + col] = acc[4 * g + v];
  __syncthreads();
  for (int e = tid; e < BM * BM; e += blockDim.x) {
    const int b = e / BM, c = e % BM, jj = jt * BM + c;
    if (jj >= r) continue;
    t_part[((size_t)ks * BM + b) * r + jj] = red[0][e] + red[1][e] + red[2][e] + red[3][e];
  }
}

// Row b of t (one block per padded row): the sum of the K-split partials (in
// order) times 1 / sx[b], then times its own row scale st[b] as fp16 hi/lo
// [32][r] in operand order.  Each thread issues all its partial loads before
// the first add.
constexpr int BT_T = 1024;
constexpr int BT_V = 4;                  // values per thread (r <= 4096)
constexpr int BT_KS = 16;                // most K splits

__global__ void __launch_bounds__(BT_T)
k_bsplit_t(const float* __restrict__ t_part, int ksplit, int r, const float* __restrict__ sx,
           _Float16* __restrict__ th, _Float16* __restrict__ tl, float* __restrict__ st) {
  __shared__ float mred[BT_T / WAVE];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const float ix = 1.f / sx[b];
  float v[BT_V];
  float mx = 0.f;
#pragma unroll
  for (int q = 0; q < BT_V; ++q) {
    const int j = min(tid + BT_T * q, r - 1);
    const size_t e = (size_t)b * r + j;
    float p[BT_KS];
#pragma unroll
    for (int ks = 0; ks < BT_KS; ++ks) p[ks] = t_part[(size_t)min(ks, ksplit - 1) * BM * r + e];
    float a = p[0];
#pragma unroll
    for (int ks = 1; ks < BT_KS; ++ks)
      if (ks < ksplit) a += p[ks];
    v[q] = a * ix;
    if (tid + BT_T * q < r) mx = fmaxf(mx, fabsf(v[q]));
  }
  mx = wave_max(mx);
  if (lane == 0) mred[w] = mx;
  __syncthreads();
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < BT_T / WAVE; ++i) m = fmaxf(m, mred[i]);
  const float sc = pow2_scale(m);
  if (tid == 0) st[b] = sc;
#pragma unroll
  for (int q = 0; q < BT_V; ++q) {
    const int j = tid + BT_T * q;
    if (j < r) {
      _Float16 hh, ll;
      split_f16(v[q] * sc, &hh, &ll);
      th[aop(b, j)] = hh;
      tl[aop(b, j)] = ll;
    }
  }
}

// ------------------------------------------------------------ predictor 2
// s[b][i] = c_i + sum_k t[b][k] B[i][k] for BS_T tiles of 32 neurons per block:
// its 4 waves split K into contiguous ranges and each multiplies its range of t
// (hi/lo, read once per block instead of once per tile) with the rows of all the
// block's tiles; the partials are summed through LDS in wave order.  Mask
// m[i][b] = (s > 0) for b < batch (0 for padded rows), one byte each in
// neuron-major layout [ffn][32]; union u[i] = OR_b m[i][b]; each tile's union
// count to cnt_blk[tile].  Optional outputs in sequence-major layout:
// scores[b][i] and mask_out[b][i].  Neurons i < hot (the hot-dense prefix) are on
// in every sequence without a score: a block wholly inside the prefix reads no
// row of B, and no score of the prefix is written.
constexpr int BS_W = 4;                  // waves (K split)

// BS_T (1..4) tiles per block, chosen by the host for an even spread over the compute units
template <int PT, int BS_T>
__global__ void __launch_bounds__(BS_W * WAVE) __attribute__((amdgpu_waves_per_eu(2)))
k_bscore(const void* __restrict__ Bm, const float* __restrict__ pbias, int f, int r, int batch,
         const _Float16* __restrict__ th, const _Float16* __restrict__ tl, const float* __restrict__ st,
         uint8_t* __restrict__ m_nm, uint8_t* __restrict__ u, int32_t* __restrict__ cnt_blk,
         float* __restrict__ scores, uint8_t* __restrict__ mask_out, int hot) {
  constexpr int KS_U = (PT == DT_F32 ? 4 : 8) / (BS_T > 1 ? 2 : 1);   // K steps per batch of loads
  static_assert(BS_T >= 1 && BS_T <= 4, "tiles per block");
  constexpr int WV = PT == DT_F32 ? 2 : 1;           // 16-byte pieces per 8 weights
  __shared__ float red[BS_W][BS_T][BM * BM];
  __shared__ uint32_t onr[BS_T][BS_W * WAVE];
  __shared__ int cnt_t[BS_T];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int col = lane % 32, half = lane / 32;
  const int i0 = blockIdx.x * BS_T * BM;
  f16v acc[BS_T];
#pragma unroll
  for (int t = 0; t < BS_T; ++t) acc[t] = f16v{};
  const int ns = r / 16, kbeg = 16 * (w * ns / BS_W), kend = 16 * ((w + 1) * ns / BS_W);
  // the epilogue's predictor biases and row scales, loaded ahead of the products
  const int c = tid % BM;
  float cbv[BS_T], stv[BM / 8];
#pragma unroll
  for (int t = 0; t < BS_T; ++t) cbv[t] = pbias[min(i0 + BM * t + c, f - 1)];
#pragma unroll
  for (int q = 0; q < BM / 8; ++q) stv[q] = st[tid / BM + 8 * q];
  if (i0 + BS_T * BM > hot) {                // block-uniform: a block wholly in the hot prefix reads no row of B
    for (int k = kbeg; k < kend; k += 16 * KS_U) {
      h8v ah[KS_U], al[KS_U];
      uint4 bv[BS_T][KS_U][WV];
#pragma unroll
      for (int uu = 0; uu < KS_U; ++uu) {
        const int ks = min(k + 16 * uu, kend - 16), kk = ks + 8 * half;
        const size_t xo = (size_t)(ks >> 4) * 512 + 8 * lane;
        ah[uu] = *reinterpret_cast<const h8v*>(th + xo);
        al[uu] = *reinterpret_cast<const h8v*>(tl + xo);
#pragma unroll
        for (int t = 0; t < BS_T; ++t) {
          const size_t row = (size_t)min(i0 + BM * t + col, f - 1);
          if constexpr (PT == DT_F16) {
            bv[t][uu][0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(Bm) + row * r + kk);
          } else {
            const float* fp = static_cast<const float*>(Bm) + row * r + kk;
            bv[t][uu][0] = *reinterpret_cast<const uint4*>(fp);
            bv[t][uu][1] = *reinterpret_cast<const uint4*>(fp + 4);
          }
        }
      }
      PI_ISSUE_FENCE();
      const h8v z8 = {};
#pragma unroll
      for (int uu = 0; uu < KS_U; ++uu) {
        const bool ok = k + 16 * uu < kend;
        const h8v a = ok ? ah[uu] : z8, l = ok ? al[uu] : z8;
#pragma unroll
        for (int t = 0; t < BS_T; ++t) {
          if constexpr (PT == DT_F16) {
            const h8v bw = as_h8(bv[t][uu][0]);
            acc[t] = mfma(a, bw, acc[t]);
            acc[t] = mfma(l, bw, acc[t]);
          } else {
            const float v[8] = {__uint_as_float(bv[t][uu][0].x), __uint_as_float(bv[t][uu][0].y),
                                __uint_as_float(bv[t][uu][0].z), __uint_as_float(bv[t][uu][0].w),
                                __uint_as_float(bv[t][uu][1].x), __uint_as_float(bv[t][uu][1].y),
                                __uint_as_float(bv[t][uu][1].z), __uint_as_float(bv[t][uu][1].w)};
            h8v bh, bl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              _Float16 hh, ll;
              split_f16(v[e], &hh, &ll);
              bh[e] = hh;
              bl[e] = ll;
            }
            acc[t] = mfma(a, bh, acc[t]);
            acc[t] = mfma(l, bh, acc[t]);
            acc[t] = mfma(a, bl, acc[t]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < BS_T; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[w][t][(8 * g + 4 * half + v) * BM + col] = acc[t][4 * g + v];
  if (tid < BS_T) cnt_t[tid] = 0;
  __syncthreads();
  // per tile, thread (neuron c = tid % 32, batch rows tid / 32 + 8 q): 256 threads
  // cover the 32 x 32 tile four rows each
#pragma unroll
  for (int t = 0; t < BS_T; ++t) {
    const int ii = i0 + BM * t + c;
    const bool col_ok = ii < f;
    const float cb = cbv[t];
    uint32_t on_rows = 0;
#pragma unroll
    for (int q = 0; q < BM / 8; ++q) {
      const int b = tid / BM + 8 * q;
      const int e = b * BM + c;
      float sacc = red[0][t][e];
#pragma unroll
      for (int v = 1; v < BS_W; ++v) sacc += red[v][t][e];
      const float sv = sacc * (1.f / stv[q]) + cb;         // the row's scale undone exactly
      const bool on = col_ok && b < batch && (ii < hot || sv > 0.f);
      on_rows |= (on ? 1u : 0u) << b;
      if (col_ok) {
        m_nm[(size_t)ii * BM + b] = on ? 1 : 0;
        if (b < batch) {
          if (scores && ii >= hot) scores[(size_t)b * f + ii] = sv;
          if (mask_out) mask_out[(size_t)b * f + ii] = on ? 1 : 0;
        }
      }
    }
    onr[t][tid] = on_rows;
  }
  __syncthreads();
  if (tid < BS_T * BM) {
    const int t = tid / BM, ii = i0 + BM * t + c;
    uint32_t all = 0;
#pragma unroll
    for (int q = 0; q < (BS_W * WAVE) / BM; ++q) all |= onr[t][c + BM * q];
    const bool un = all != 0;
    if (ii < f) u[ii] = un ? 1 : 0;
    if (ii < f && un) atomicAdd(&cnt_t[t], 1);   // LDS atomic
  }
  __syncthreads();
  if (tid < BS_T && cnt_blk) {
    const int tile = blockIdx.x * BS_T + tid;
    if (tile < (f + BM - 1) / BM) cnt_blk[tile] = cnt_t[tid];
  }
}

// The rows the batched FFN runs over: the union list, or -- when the union
// holds at least dense_min neurons -- every neuron in storage order (a dense
// GEMM; neurons outside the union get h = 0 from their all-zero mask bytes).
// Both FFN kernels take the same decision from the same device-resident count.
__device__ __forceinline__ int ffn_rows(const int32_t* __restrict__ ucount, int f, int dense_min, bool* dense) {
  const int n = min(max(*ucount, 0), f);
  *dense = n >= dense_min;
  return *dense ? f : n;
}

// ------------------------------------------------------------ up / gate
// z = X W^T over the union rows (fp16 and fp32 weights).  A block takes tiles
// q = blockIdx.x, blockIdx.x + gridDim.x, ... of 32 union list entries [32 q,
// 32 q + 32) while they exist; its bup_waves(NMAT) waves split K
// into contiguous ranges and their partial tiles are summed through LDS in
// wave order.  Epilogue: z's row b times 1 / sx[b]; h[b] = m[i][b] ?
// act(z + bias) : 0, written in fp32 to h32 as a [32][h_stride] operand-order
// matrix (row b, column j = the neuron's position in the union list), in which
// the down projection reads it as its A operand; hmax[b] collects the largest
// |h[b]| (as the bits of a non-negative float, by atomic maximum).
// waves per block: 8, or 4 for ReGLU (two z tiles per wave in the LDS sum, so that
// four blocks fit on a compute unit; 66.1 -> 60.7 us at the LLaMA-2-7B shape, batch 32)
__host__ __device__ constexpr int bup_waves(int nmat) { return nmat == 2 ? 4 : 8; }
constexpr int BD_CH = 128;               // union positions per chunk of the down projection

// K extent (halves) of the h operand: whole chunks, so that a chunk's
// reads stay inside the buffer
__host__ __device__ constexpr int h_stride(int f) { return (f + BD_CH - 1) / BD_CH * BD_CH; }

template <int WT, int ACT>
__global__ void __launch_bounds__(bup_waves(act_nmat<ACT>()) * WAVE)
k_bup(const void* __restrict__ gate_w, const uint16_t* __restrict__ gate_sc, const void* __restrict__ up_w,
      const uint16_t* __restrict__ up_sc, const float* __restrict__ bias, int f, int d,
      const _Float16* __restrict__ xh, const _Float16* __restrict__ xl, const int32_t* __restrict__ ulist,
      const int32_t* __restrict__ ucount, const uint8_t* __restrict__ m_nm, const float* __restrict__ sx,
      float* __restrict__ h32, uint32_t* __restrict__ hmax, int dense_min) {
  constexpr int NMAT = act_nmat<ACT>();
  constexpr int BUP_W = bup_waves(NMAT);
  __shared__ float red[BUP_W][NMAT][BM * BM];
  __shared__ uint32_t rmax[BM];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int col = lane % 32, half = lane / 32;
  bool dense;
  const int n = ffn_rows(ucount, f, dense_min, &dense);
  // union tiles blockIdx.x, blockIdx.x + gridDim.x, ... (the grid is sized for the
  // chip, the tile count is on the device)
  for (int tile = blockIdx.x; tile * BM < n; tile += gridDim.x) {
    const int t0 = tile * BM;
    const int row = dense ? min(t0 + col, n - 1) : ulist[min(t0 + col, n - 1)];
    f16v acc[NMAT];
#pragma unroll
    for (int mt = 0; mt < NMAT; ++mt) acc[mt] = f16v{};
    const int ns = d / 16, kbeg = 16 * (w * ns / BUP_W), kend = 16 * ((w + 1) * ns / BUP_W);
    for (int k = kbeg; k < kend; k += 16 * KU) {
#pragma unroll
      for (int mt = 0; mt < NMAT; ++mt)
        mfma_window<WT>(acc[mt], xh, xl, (NMAT == 2 && mt == 0) ? gate_w : up_w, (size_t)row, d, k, kend, 16, lane);
    }
    // the waves' partial tiles: lane holds neuron column col, batch rows 8g + 4*half + v
#pragma unroll
    for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[w][mt][(8 * g + 4 * half + v) * BM + col] = acc[mt][4 * g + v];
    if (tid < BM) rmax[tid] = 0u;
    __syncthreads();
    for (int e = tid; e < BM * BM; e += blockDim.x) {
      const int b = e / BM, c = e % BM;
      if (t0 + c >= n) continue;
      const float ix = 1.f / sx[b];
      float z[NMAT];
#pragma unroll
      for (int mt = 0; mt < NMAT; ++mt) {
        float s = 0.f;
#pragma unroll
        for (int v = 0; v < BUP_W; ++v) s += red[v][mt][e];
        z[mt] = s * ix;
      }
      const int rw = dense ? t0 + c : ulist[t0 + c];
      float h = act_h<ACT>(z[0], bias[rw], z[NMAT - 1]);
      if (m_nm[(size_t)rw * BM + b] == 0) h = 0.f;
      h32[aop(b, t0 + c)] = h;
      atomicMax(&rmax[b], __float_as_uint(fabsf(h)));         // LDS atomic
    }
    __syncthreads();
    if (tid < BM && rmax[tid] != 0u) atomicMax(&hmax[tid], rmax[tid]);
    __syncthreads();                                            // red and rmax are reused by the next tile
  }
}

// ---------------------------------------------- up / gate, K-split (Q4_0)
// z = X W^T over the union rows with the batch operand staged in LDS once per
// block and used for BU_TPB row tiles.  Work item g KS + s: row tiles
// [g BU_TPB, (g + 1) BU_TPB) of the union list and K split s (the items of
// one split land on one XCD when KS = 8, so its X slice stays in that L2).
// The split's K range is walked in chunks of KC: the chunk of X (fp16 hi and
// lo, operand order) goes to LDS by LDS-DMA while each wave loads its weights
// for it; wave w takes row tile w % BU_TPB and half w / BU_TPB of the chunk.
// The two halves' tiles are added in LDS, and the split's partial z goes to
// z_part[s][m][position][b] (b fastest).  k_bup_epi adds the splits in order
// and applies the activation.
constexpr int BU_TPB = 4;                // row tiles (32 union rows each) per block
constexpr int BU_KSMAX = 8;              // K splits (partial z vectors)
__host__ __device__ constexpr int bu_kc(int nmat) { return 512 / nmat; }   // K per staged chunk
// K splits for width d: the largest power of two <= BU_KSMAX that leaves whole chunks of
// 64 values per split
__host__ __device__ constexpr int bu_ks(int d) {
  return (d % (8 * 64) == 0) ? 8 : (d % (4 * 64) == 0) ? 4 : (d % (2 * 64) == 0) ? 2 : 1;
}

template <int WT, int NMAT>
__global__ void __launch_bounds__(512)
k_bup2(const void* __restrict__ gate_w, const uint16_t* __restrict__ gate_sc, const void* __restrict__ up_w,
       const uint16_t* __restrict__ up_sc, int f, int d, int KS, const _Float16* __restrict__ xh,
       const _Float16* __restrict__ xl, const int32_t* __restrict__ ulist, const int32_t* __restrict__ ucount,
       int dense_min, float* __restrict__ z_part) {
  static_assert(WT == DT_Q4, "fp16 and fp32 weights take k_bup (one pass over K measured faster)");
  constexpr int KC = bu_kc(NMAT), KH = KC / 2;      // chunk, and the half a wave takes
  static_assert(KH % 32 == 0, "whole Q4_0 blocks per half chunk");
  __shared__ __attribute__((aligned(16))) _Float16 xs[2][bu_kc(1) / 16 * 512];   // hi, lo [K step][512]
  float* red = reinterpret_cast<float*>(&xs[0][0]);                       // after the chunks: [8][NMAT][BM*BM]
  static_assert(sizeof(float) * 8 * NMAT * BM * BM <= sizeof(xs), "red fits");
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int col = lane % 32, half = lane / 32;
  bool dense;
  const int n = ffn_rows(ucount, f, dense_min, &dense);
  // items blockIdx.x, blockIdx.x + gridDim.x, ... while their row tiles exist: item
  // g KS + s is row-tile group g and K split s (gridDim.x is a multiple of KS, so
  // a block keeps its split and its XCD)
  for (int item = blockIdx.x; (item / KS) * BU_TPB * BM < n; item += gridDim.x) {
    const int g = item / KS, s = item % KS;
    const int t0 = g * BU_TPB * BM;
    const int tl = w % BU_TPB, kp = w / BU_TPB;                 // this wave's row tile and chunk half
    const int pos = min(t0 + tl * BM + col, n - 1);
    const size_t row = (size_t)(dense ? pos : ulist[pos]);
    const int ksz = d / KS, kbeg = s * ksz;
    f16v acc[NMAT];
#pragma unroll
    for (int mt = 0; mt < NMAT; ++mt) acc[mt] = f16v{};
    for (int kc = kbeg; kc < kbeg + ksz; kc += KC) {
      const int kcn = min(KC, kbeg + ksz - kc);                 // a multiple of 64
      // the chunk of X: K steps kc/16 .. (kc + kcn)/16 of hi and lo, 1 KB each
      __syncthreads();                                          // the previous chunk is consumed
      for (int p = w; p < 2 * (kcn / 16); p += 8) {
        const int hl = p & 1, st = p >> 1;
        const _Float16* src = (hl ? xl : xh) + (size_t)(kc / 16 + st) * 512;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + 8 * lane),
                                         (__attribute__((address_space(3))) void*)(&xs[hl][st * 512]), 16, 0, 0);
      }
      const int kw = kc + kp * (kcn / 2), kwn = kcn / 2;        // this wave's half
      constexpr int QB = KH / 32;
      // the row's nibbles for the half chunk (one 16-byte block per load; the two lane
      // halves hold the same rows and load alternate blocks) and its block scales two
      // at a time: aligned words from the even block a0 = kw / 32 rounded down (d / 32
      // is even, so a word lies wholly inside the row or wholly past it, then clamped
      // to the row's last word and not used); block kw / 32 + qb is half (o + qb) & 1
      // of word (o + qb) / 2, o = kw / 32 - a0
      const int a0 = (kw / 32) & ~1, o = (kw / 32) & 1;
      static_assert(QB % 2 == 0, "blocks in pairs");
      uint4 cq[NMAT][QB / 2];     // block 2m + half of the pair m (exchanged by q4_pair)
      uint32_t scw[NMAT][QB / 2 + 1];
#pragma unroll
      for (int mt = 0; mt < NMAT; ++mt) {
        const void* wp = (NMAT == 2 && mt == 0) ? gate_w : up_w;
        const uint16_t* sp = (NMAT == 2 && mt == 0) ? gate_sc : up_sc;
#pragma unroll
        for (int m = 0; m < QB / 2; ++m) {
          const int kb = kw + 32 * min(2 * m + half, kwn / 32 - 1);
          cq[mt][m] = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(wp) + row * (d / 2) + kb / 2);
        }
#pragma unroll
        for (int p = 0; p <= QB / 2; ++p)
          scw[mt][p] = *reinterpret_cast<const uint32_t*>(sp + row * (d / 32) + min(a0 + 2 * p, d / 32 - 2));
      }
      PI_ISSUE_FENCE();
      wait_vm_lds<0>();
      __syncthreads();                                        // every wave's part of the chunk is in LDS
      uint2 cw[NMAT][QB];                                     // this half's 8 bytes of each block
#pragma unroll
      for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
        for (int m = 0; m < QB / 2; ++m) q4_pair(cq[mt][m], cw[mt][2 * m], cw[mt][2 * m + 1]);
      // every block of the half chunk is multiplied (blocks past a short last
      // chunk read clamped weights and LDS steps inside xs, and are dropped by a
      // select): a branch around the use would sink the loads into it, one HBM
      // round trip per block
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const bool valid = 32 * qb < kwn;
        const int st0 = (kw - kc) / 16 + 2 * min(qb, kwn / 32 - 1);   // K step within the chunk
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt) {
          f16v p = {};
#pragma unroll
          for (int stp = 0; stp < 2; ++stp) {
            const h8v bw = q4_h8w(cw[mt][qb].x, cw[mt][qb].y, stp == 1);
            const h8v ah = *reinterpret_cast<const h8v*>(&xs[0][(st0 + stp) * 512 + 8 * lane]);
            const h8v al = *reinterpret_cast<const h8v*>(&xs[1][(st0 + stp) * 512 + 8 * lane]);
            p = mfma(ah, bw, p);
            p = mfma(al, bw, p);
          }
          const uint32_t wd = o ? scw[mt][(qb + 1) / 2] : scw[mt][qb / 2];
          const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd >> (16 * ((o + qb) & 1))));
#pragma unroll
          for (int x = 0; x < 16; ++x) acc[mt][x] = valid ? fmaf(sc, p[x], acc[mt][x]) : acc[mt][x];
        }
      }
    }
    __syncthreads();                                            // the last chunk is consumed: reuse its LDS
#pragma unroll
    for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[((size_t)w * NMAT + mt) * BM * BM + (8 * g4 + 4 * half + v) * BM + col] = acc[mt][4 * g4 + v];
    __syncthreads();
    // the two halves of each tile, in order, to z_part[s][mt][position][b]
    const size_t fpad = (size_t)(f + BM - 1) / BM * BM;
    for (int e = tid; e < BU_TPB * NMAT * BM * BM; e += blockDim.x) {
      const int b = e % BM, c = (e / BM) % BM, mt = (e / (BM * BM)) % NMAT, t = e / (NMAT * BM * BM);
      const int p = t0 + t * BM + c;
      if (p >= n) continue;
      const float v = red[((size_t)t * NMAT + mt) * BM * BM + b * BM + c] +
                      red[((size_t)(t + BU_TPB) * NMAT + mt) * BM * BM + b * BM + c];
      z_part[(((size_t)s * NMAT + mt) * fpad + p) * BM + b] = v;
    }
    __syncthreads();                                            // red is the next item's chunk buffer
  }
}

// h from the K splits of z: position j of the union list (8 per block step), row b
// (b fastest): z = (sum of the KS partials in split order) / sx[b]; h = m ? act(z
// + bias) : 0, written in fp32 to h32 in operand order; hmax[b] collects the
// largest |h[b]|.
template <int ACT>
__global__ void __launch_bounds__(256)
k_bup_epi(const float* __restrict__ z_part, int KS, int f, const int32_t* __restrict__ ulist,
          const int32_t* __restrict__ ucount, int dense_min, const float* __restrict__ bias,
          const uint8_t* __restrict__ m_nm, const float* __restrict__ sx, float* __restrict__ h32,
          uint32_t* __restrict__ hmax) {
  constexpr int NMAT = act_nmat<ACT>();
  __shared__ uint32_t rmax[BM];
  const int tid = threadIdx.x, b = tid % BM;
  bool dense;
  const int n = ffn_rows(ucount, f, dense_min, &dense);
  if (tid < BM) rmax[tid] = 0u;
  __syncthreads();
  const size_t fpad = (size_t)(f + BM - 1) / BM * BM;
  const float ix = 1.f / sx[b];
  // positions 8 q .. 8 q + 7 for q = blockIdx.x, blockIdx.x + gridDim.x, ...; all
  // BU_KSMAX partials of a value loaded before the first add (splits past KS read
  // split 0 and are dropped)
  for (int q = blockIdx.x; q * (256 / BM) < n; q += gridDim.x) {
    const int j = q * (256 / BM) + tid / BM;
    if (j < n) {
      const int rw = dense ? j : ulist[j];
      float z[NMAT];
#pragma unroll
      for (int mt = 0; mt < NMAT; ++mt) {
        float pz[BU_KSMAX];
#pragma unroll
        for (int s2 = 0; s2 < BU_KSMAX; ++s2)
          pz[s2] = z_part[(((size_t)(s2 < KS ? s2 : 0) * NMAT + mt) * fpad + j) * BM + b];
        float a = pz[0];
#pragma unroll
        for (int s2 = 1; s2 < BU_KSMAX; ++s2) a += s2 < KS ? pz[s2] : 0.f;
        z[mt] = a * ix;
      }
      float h = act_h<ACT>(z[0], bias[rw], z[NMAT - 1]);
      if (m_nm[(size_t)rw * BM + b] == 0) h = 0.f;
      h32[aop(b, j)] = h;
      atomicMax(&rmax[b], __float_as_uint(fabsf(h)));          // LDS atomic
    }
  }
  __syncthreads();
  if (tid < BM && rmax[tid] != 0u) atomicMax(&hmax[tid], rmax[tid]);
}

// ------------------------------------------------------ union compaction
// The ascending union list from the score kernel's per-tile union bytes u and
// counts (one per 32-neuron tile), in one pass without atomics: block b takes
// tiles [256 b, 256 b + 256); it adds the counts of all earlier tiles (a few KB
// read from L2) and scans its own, and each thread writes the union neurons of
// one tile at its offset.  Every load is issued before the first use, so the
// kernel is one round trip.  *count (and count2, count3 if given) = the total,
// from block 0 (which adds every tile's count).
__global__ void __launch_bounds__(256)
k_bcompact(const uint8_t* __restrict__ u, const int32_t* __restrict__ tile_cnt, int f, int32_t* __restrict__ list,
           int32_t* __restrict__ count, int32_t* __restrict__ count2, int32_t* __restrict__ count3) {
  constexpr int BC_PRE = 8;                  // earlier tile counts per thread (f <= 65536: 2048 tiles)
  __shared__ int red[2][4];
  __shared__ int wtot[4];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int ntiles = (f + BM - 1) / BM;
  const int t0 = blockIdx.x * 256, t = t0 + tid;
  // every load first: the earlier tiles' counts (block 0: all counts, for the
  // total), this tile's count and its 32 union bytes
  const int span = blockIdx.x == 0 ? ntiles : t0;
  int pre[BC_PRE];
#pragma unroll
  for (int q = 0; q < BC_PRE; ++q) {
    const int k = tid + 256 * q;
    pre[q] = k < span ? tile_cnt[k] : 0;
  }
  const int c = t < ntiles ? tile_cnt[t] : 0;
  uint4 ub[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
  if (t < ntiles && (t + 1) * BM <= f) {
    ub[0] = reinterpret_cast<const uint4*>(u + (size_t)t * BM)[0];
    ub[1] = reinterpret_cast<const uint4*>(u + (size_t)t * BM)[1];
  }
  int sp = 0;
#pragma unroll
  for (int q = 0; q < BC_PRE; ++q) sp += pre[q];
  sp = wave_sum(sp);
  const int inc = wave_scan(c);
  if (lane == 0) red[0][w] = sp;
  if (lane == WAVE - 1) wtot[w] = inc;
  __syncthreads();
  const int spb = red[0][0] + red[0][1] + red[0][2] + red[0][3];   // block 0: the total
  const int before = blockIdx.x == 0 ? 0 : spb;
  int off = before + inc - c;
  for (int v = 0; v < w; ++v) off += wtot[v];
  if (t < ntiles && c > 0) {
    const int i0 = t * BM;
    if (i0 + BM <= f) {
      const uint32_t wd[8] = {ub[0].x, ub[0].y, ub[0].z, ub[0].w, ub[1].x, ub[1].y, ub[1].z, ub[1].w};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if ((wd[q] >> (8 * e)) & 0xFFu) list[off++] = i0 + 4 * q + e;
      }
    } else {
      for (int k = 0; k < f - i0; ++k)                        // the ragged last tile, bytewise
        if (u[i0 + k]) list[off++] = i0 + k;
    }
  }
  if (blockIdx.x == 0 && tid == 0) {
    *count = spb;
    if (count2) *count2 = spb;
    if (count3) *count3 = spb;
  }
}

// ------------------------------------------------------------------ down
// y[b][c] = sum over union positions j of h[b][j] downT[u_j][c].  Block =
// one group of BD_COLS = 256 columns (wave w owns the 32-column tile w) and
// one of bd_splits(d) splits of the union list; a split's share is taken in
// chunks of BD_CH positions, and its partial sums go to y_part[split][b][c]
// (b < batch; the consumer adds the splits in order, b_down rides on split 0).
// Per chunk the block stages, in LDS,
//  - the A operands once for all eight tiles: h (read in its operand-order
//    layout) times the row scale from hmax, split into fp16 hi/lo;
//  - each tile's weights transposed to [column][position] as fp16 hi + lo
//    pairs.
// k_bdown takes fp32 weights: every thread converts four positions of eight
// columns in each of its two items (adjacent tiles) and writes each column's
// values in pairs; the next chunk's weights and h, and the row ids of the chunk
// after it, are in flight while a chunk is converted and multiplied.  Blocks
// read a whole 128-byte line (or several) of every row they gather, and h once
// per 256 columns instead of once per 32 or 64.  Q4_0 and fp16 weights take
// k_bdown_q4 and k_bdown_f16 (same blocks and chunks, more chunks in flight).
constexpr int BD_COLS = 256;             // columns per block (eight 32-column tiles, one per wave)
constexpr int BD_PAD = BD_CH + 8;        // padded position stride (halves) of a transposed column
constexpr int BD_MAXSPLIT = 16;          // most splits of the union list (partial y vectors)
constexpr int BD_MAXF = 65536;           // largest ffn of the batched path
// splits of the union list for width d: about one block per compute unit
__host__ __device__ constexpr int bd_splits(int d) {
  return (256 / ((d + BD_COLS - 1) / BD_COLS)) < 1 ? 1
         : (256 / ((d + BD_COLS - 1) / BD_COLS)) > BD_MAXSPLIT ? BD_MAXSPLIT
                                                              : 256 / ((d + BD_COLS - 1) / BD_COLS);
}

template <int WT>
__global__ void __launch_bounds__(512)
k_bdown(const void* __restrict__ downT, int f, int d, const int32_t* __restrict__ ulist,
        const int32_t* __restrict__ ucount, const float* __restrict__ h32, const uint32_t* __restrict__ hmax,
        const float* __restrict__ b_down, int batch, float* __restrict__ y_part, int dense_min, int nsplit) {
  static_assert(WT == DT_F32, "Q4_0 and fp16 weights take k_bdown_q4 and k_bdown_f16");
  constexpr int NW = 2;                            // weight operands: hi and lo
  constexpr int NWV = 4;                           // 16-byte pieces per row segment of 8 columns, times items
  __shared__ __attribute__((aligned(16))) _Float16 wt[NW][BD_COLS][BD_PAD];
  __shared__ __attribute__((aligned(16))) _Float16 as[2][BD_CH / 16][512];
  __shared__ float rsc[BM];                        // 1 / row scale of h, per batch row
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int ngroup = (d + BD_COLS - 1) / BD_COLS;
  const int c0 = (int)(blockIdx.x % ngroup) * BD_COLS, split = (int)blockIdx.x / ngroup;
  bool dense;
  const int n = ffn_rows(ucount, f, dense_min, &dense);
  const int nch_all = (n + BD_CH - 1) / BD_CH, cps = (nch_all + nsplit - 1) / nsplit;
  const int ch0 = split * cps;                     // this split's chunks [ch0, ch0 + nch)
  const int nch = max(0, min(nch_all, ch0 + cps) - ch0);
  const int pg = tid & 31;                         // staging: chunk positions 4 pg .. 4 pg + 3
  const float hs = pow2_scale(__uint_as_float(hmax[lane & 31]));   // A staging: this lane's batch row
  if (tid < BM) rsc[tid] = 1.f / pow2_scale(__uint_as_float(hmax[tid]));
  f16v acc = {};

  // the row ids of chunk c's positions 4 pg + q (clamped into the list)
  auto load_ids = [&](int c, int (&id)[4]) __attribute__((always_inline)) {
    const int base = (ch0 + c) * BD_CH;
#pragma unroll
    for (int q = 0; q < 4; ++q) id[q] = ulist[max(0, min(base + 4 * pg + q, n - 1))];
  };
  // Items of a thread: i = 0, 1 are the adjacent tiles 2 (t >> 7) + i (t = tid), in
  // both at columns 8 cq .. 8 cq + 7 with cq = (t >> 5) & 3.
  struct Stage {
    uint4 wv[2][4][NWV / 2];  // items x four rows: the 32 bytes of each row segment
    float4 hv[2];             // 8 values of h for the A operands
  };
  auto fetch = [&](int c, const int (&id)[4], Stage& st) __attribute__((always_inline)) {
    const int base = (ch0 + c) * BD_CH;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const size_t row = (size_t)(dense ? max(0, min(base + 4 * pg + q, n - 1)) : id[q]);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int tile = 2 * (tid >> 7) + i;
        const int col = min(c0 + BM * tile + 8 * ((tid >> 5) & 3), d - 8);
        const float* fp = static_cast<const float*>(downT) + row * d + col;
        st.wv[i][q][0] = *reinterpret_cast<const uint4*>(fp);
        st.wv[i][q][1] = *reinterpret_cast<const uint4*>(fp + 4);
      }
    }
    const float4* hp = reinterpret_cast<const float4*>(h32 + (size_t)((ch0 + c) * (BD_CH / 16) + w) * 512 + 8 * lane);
    st.hv[0] = hp[0];
    st.hv[1] = hp[1];
  };
  // a chunk's operands into LDS; positions past the list end and columns past d are zero
  // (h there is whatever an earlier call left: 0 * NaN is not zero)
  auto convert = [&](const Stage& st, int c) __attribute__((always_inline)) {
    const int base = (ch0 + c) * BD_CH;
    typedef _Float16 h4v __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int tile = 2 * (tid >> 7) + i, cq = (tid >> 5) & 3;
      const bool okc = c0 + BM * tile + 8 * cq < d;
      _Float16* dst0 = &wt[0][BM * tile + 8 * cq][4 * pg];
      float v[4][8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool ok = okc && c < nch && base + 4 * pg + q < n;
        const float a8[8] = {__uint_as_float(st.wv[i][q][0].x), __uint_as_float(st.wv[i][q][0].y),
                             __uint_as_float(st.wv[i][q][0].z), __uint_as_float(st.wv[i][q][0].w),
                             __uint_as_float(st.wv[i][q][1].x), __uint_as_float(st.wv[i][q][1].y),
                             __uint_as_float(st.wv[i][q][1].z), __uint_as_float(st.wv[i][q][1].w)};
#pragma unroll
        for (int e = 0; e < 8; ++e) v[q][e] = ok ? a8[e] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        _Float16 hi[4], lo[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) split_f16(v[q][e], &hi[q], &lo[q]);
        *reinterpret_cast<h4v*>(dst0 + e * BD_PAD) = h4v{hi[0], hi[1], hi[2], hi[3]};
        *reinterpret_cast<h4v*>(&wt[NW - 1][BM * tile + 8 * cq + e][4 * pg]) = h4v{lo[0], lo[1], lo[2], lo[3]};
      }
    }
    // A operands: K step w of the chunk, operand slot lane (batch row lane % 32)
    const int jj = base + 16 * w + 8 * (lane / 32);
    const float hv8[8] = {st.hv[0].x, st.hv[0].y, st.hv[0].z, st.hv[0].w,
                          st.hv[1].x, st.hv[1].y, st.hv[1].z, st.hv[1].w};
    h8v ahi, alo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      _Float16 hi, lo;
      split_f16(c < nch && jj + e < n ? hv8[e] * hs : 0.f, &hi, &lo);
      ahi[e] = hi;
      alo[e] = lo;
    }
    *reinterpret_cast<h8v*>(&as[0][w][8 * lane]) = ahi;
    *reinterpret_cast<h8v*>(&as[1][w][8 * lane]) = alo;
  };

  // chunk c: the next chunk's loads, its operands into LDS, the products.  No
  // branch: the loop runs whole pairs of chunks, a chunk past the split's end
  // converts to zeros, and the loads past the end repeat the last chunk
  // (clamped) -- a branch around a use lets the compiler sink loads and
  // operand math into it, after the next chunk's loads, and then wait for
  // those too.
  auto step = [&](const Stage& cur, Stage& nxt, const int (&id_next)[4], int (&id_after)[4], int c)
      __attribute__((always_inline)) {
    fetch(min(c + 1, nch - 1), id_next, nxt);      // in flight while this chunk is converted and multiplied
    convert(cur, c);
    load_ids(min(c + 2, nch - 1), id_after);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < BD_CH / 16; ++ks) {
      const int kb = 16 * ks + 8 * (lane / 32);
      const h8v ah = *reinterpret_cast<const h8v*>(&as[0][ks][8 * lane]);
      const h8v al = *reinterpret_cast<const h8v*>(&as[1][ks][8 * lane]);
      const h8v bw = *reinterpret_cast<const h8v*>(&wt[0][BM * w + (lane & 31)][kb]);
      acc = mfma(ah, bw, acc);
      acc = mfma(al, bw, acc);
      const h8v bl = *reinterpret_cast<const h8v*>(&wt[1][BM * w + (lane & 31)][kb]);
      acc = mfma(ah, bl, acc);
    }
    __syncthreads();
  };
  int id_a[4], id_b[4];
  Stage s0, s1;
  if (nch > 0) {
    load_ids(0, id_a);
    fetch(0, id_a, s0);
    load_ids(min(1, nch - 1), id_b);
  }
  for (int c = 0; c < nch; c += 2) {
    step(s0, s1, id_b, id_a, c);
    step(s1, s0, id_a, id_b, c + 1);
  }
  __syncthreads();                                 // rsc is written
  // lane holds column c0 + 32 w + lane % 32, batch rows 8 g + 4 (lane / 32) + v
  const int cg = c0 + BM * w + (lane & 31);
  if (cg < d) {
    const float bd = (b_down && split == 0) ? b_down[cg] : 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int b = 8 * g + 4 * (lane / 32) + v;
        if (b < batch) y_part[((size_t)split * BM + b) * d + cg] = acc[4 * g + v] * rsc[b] + bd;
      }
  }
}

// ------------------------------------------------- down projection (Q4_0)
// k_bdown's blocks, splits and chunks for Q4_0 weights, organised for
// memory-level parallelism.  Thread t of the block takes chunk positions
// 16 (t / 64) + 2 r and + 1 (r = (t % 64) / 8) of tile q = t % 8: eight lanes
// read the 128 bytes of a row's segment (one line per row, not one per lane),
// every 16-byte Q4_0 block is loaded once, and each column's pair of
// positions is one 4-byte LDS write.  A column's positions are stored in
// 16-byte groups (8 positions) with group g at g ^ 2 (c / 32 % 8): the 64 lanes
// of a write then hit 64 different banks, and a wave's MFMA reads (one tile,
// one XOR value) are as without the swizzle.  The weights enter as hi = fl16(q s)
// and lo = fl16(q s - hi) with (q - 8) exact in fp16 (q s - hi has at most 4
// significant bits).  Three chunks are in flight while one is converted and
// multiplied.  Loads complete in issue order, so the row ids of a chunk are
// loaded two steps before its weights, first in their step: the wait for them
// then covers only the chunk that is converted in that same step.
__host__ __device__ constexpr int bdq_slot(int col, int pos) {   // halves offset of (col, pos) in a wt plane
  return col * BD_PAD + 8 * ((pos / 8) ^ (2 * ((col / BM) % 8))) + pos % 8;
}

__global__ void __launch_bounds__(512)
k_bdown_q4(const uint8_t* __restrict__ downT, const uint16_t* __restrict__ down_sc, int f, int d,
           const int32_t* __restrict__ ulist, const int32_t* __restrict__ ucount, const float* __restrict__ h32,
           const uint32_t* __restrict__ hmax, const float* __restrict__ b_down, int batch,
           float* __restrict__ y_part, int dense_min, int nsplit) {
  __shared__ __attribute__((aligned(16))) _Float16 wt[2][BD_COLS * BD_PAD];
  __shared__ __attribute__((aligned(16))) _Float16 as[2][BD_CH / 16][512];
  __shared__ float rsc[BM];
  static_assert(BD_CH == 128 && BD_COLS == 8 * BM, "16 positions per wave, 8 tiles per block");
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int ngroup = (d + BD_COLS - 1) / BD_COLS;
  // consecutive launch indices go to the 8 XCDs in turn: each XCD takes a run of
  // consecutive (split, column group) items, so the column groups that share a
  // line of a row's block scales, and the blocks that share a split's h, meet in
  // one L2
  const int nblk = (int)gridDim.x;
  const int L = nblk % 8 == 0 ? (int)(blockIdx.x % 8) * (nblk / 8) + (int)blockIdx.x / 8 : (int)blockIdx.x;
  const int c0 = (L % ngroup) * BD_COLS, split = L / ngroup;
  bool dense;
  const int n = ffn_rows(ucount, f, dense_min, &dense);
  const int nch_all = (n + BD_CH - 1) / BD_CH, cps = (nch_all + nsplit - 1) / nsplit;
  const int ch0 = split * cps;
  const int nch = max(0, min(nch_all, ch0 + cps) - ch0);
  const float hs = pow2_scale(__uint_as_float(hmax[lane & 31]));
  if (tid < BM) rsc[tid] = 1.f / pow2_scale(__uint_as_float(hmax[tid]));
  // this thread's tile (its Q4_0 block in every row, clamped into the row when the
  // tile is past d, then dropped), the aligned word of two block scales that holds
  // its scale (half q & 1: c0 / 32 is a multiple of 8, d / 32 even), its positions
  const int q = tid & 7, p0 = 16 * w + 2 * ((tid & 63) >> 3);
  const bool okc = c0 + BM * q < d;
  const int cb = min(c0 + BM * q, d - BM);
  const int sw = min(c0 / 32 + (q & ~1), d / 32 - 2);
  const int ssh = 16 * (q & 1);
  f16v acc = {};

  struct Stage {
    uint4 wv[2];      // the tile's block of the rows at positions p0, p0 + 1
    uint32_t sc[2];   // their scale words
    float4 hv[2];     // 8 values of h for the A operands
  };
  // chunk c's rows at positions p0 + k (clamped into the list and the split)
  // (the dense and the list case are separate instantiations of the loop below:
  // any select between a loaded id and a position is placed by the compiler next
  // to the load, with a wait for every load before it)
  auto load_ids = [&](auto dense_c, int c, int (&id)[2]) __attribute__((always_inline)) {
    const int base = (ch0 + min(c, nch - 1)) * BD_CH + p0;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int p = max(0, min(base + k, n - 1));
      id[k] = decltype(dense_c)::value ? p : ulist[p];
    }
  };
  auto fetch = [&](int c, const int (&id)[2], Stage& st) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const size_t row = (size_t)id[k];
      st.wv[k] = *reinterpret_cast<const uint4*>(downT + row * (d / 2) + cb / 2);
      st.sc[k] = *reinterpret_cast<const uint32_t*>(down_sc + row * (d / 32) + sw);
    }
    const float4* hp =
        reinterpret_cast<const float4*>(h32 + (size_t)((ch0 + min(c, nch - 1)) * (BD_CH / 16) + w) * 512 + 8 * lane);
    st.hv[0] = hp[0];
    st.hv[1] = hp[1];
  };
  // a chunk's operands into LDS; positions past the split or the list and columns
  // past d are zero (a zero scale; h there is whatever an earlier call left)
  auto convert = [&](const Stage& st, int c) __attribute__((always_inline)) {
    const int base = (ch0 + c) * BD_CH;
    const uint32_t m0 = 0u - (uint32_t)(okc && c < nch && base + p0 < n);
    const uint32_t m1 = 0u - (uint32_t)(okc && c < nch && base + p0 + 1 < n);
    const h2v s2 = {__builtin_bit_cast(_Float16, (uint16_t)((st.sc[0] >> ssh) & m0)),
                    __builtin_bit_cast(_Float16, (uint16_t)((st.sc[1] >> ssh) & m1))};
    const h2v off = {(_Float16)1032.f, (_Float16)1032.f};
    _Float16* dh = &wt[0][bdq_slot(BM * q, p0)];
    _Float16* dl = &wt[1][bdq_slot(BM * q, p0)];
    const uint32_t a[4] = {st.wv[0].x, st.wv[0].y, st.wv[0].z, st.wv[0].w};
    const uint32_t b[4] = {st.wv[1].x, st.wv[1].y, st.wv[1].z, st.wv[1].w};
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // byte j of word k (columns 4 k + j, low nibble, and 4 k + j + 16, high
        // nibble) of both rows, in the low bytes of two 16-bit lanes
        const uint32_t p = __builtin_amdgcn_perm(b[k], a[k], 0x0c000c00u | (uint32_t)j | ((uint32_t)(4 + j) << 16));
        const h2v ql = __builtin_bit_cast(h2v, (p & 0x000F000Fu) | 0x64006400u) - off;
        const h2v qh = __builtin_bit_cast(h2v, ((p >> 4) & 0x000F000Fu) | 0x64006400u) - off;
        const h2v hl = ql * s2, hh = qh * s2;
        const h2v ll = __builtin_elementwise_fma(ql, s2, -hl), lh = __builtin_elementwise_fma(qh, s2, -hh);
        const int e = 4 * k + j;   // columns of one tile share the swizzle: a column's offset is e BD_PAD
        *reinterpret_cast<h2v*>(dh + e * BD_PAD) = hl;
        *reinterpret_cast<h2v*>(dl + e * BD_PAD) = ll;
        *reinterpret_cast<h2v*>(dh + (e + 16) * BD_PAD) = hh;
        *reinterpret_cast<h2v*>(dl + (e + 16) * BD_PAD) = lh;
      }
    // A operands: K step w of the chunk, operand slot lane (batch row lane % 32)
    const int jj = base + 16 * w + 8 * (lane / 32);
    const float hv8[8] = {st.hv[0].x, st.hv[0].y, st.hv[0].z, st.hv[0].w,
                          st.hv[1].x, st.hv[1].y, st.hv[1].z, st.hv[1].w};
    h8v ahi, alo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      _Float16 hi, lo;
      split_f16(c < nch && jj + e < n ? hv8[e] * hs : 0.f, &hi, &lo);
      ahi[e] = hi;
      alo[e] = lo;
    }
    *reinterpret_cast<h8v*>(&as[0][w][8 * lane]) = ahi;
    *reinterpret_cast<h8v*>(&as[1][w][8 * lane]) = alo;
  };
  // chunk c: the row ids of chunk c + 5, the loads of chunk c + 3, then chunk c's
  // operands and products.  Loads past the split repeat its last chunk.
  auto step = [&](auto dense_c, int c, const Stage& cur, Stage& far, const int (&id_far)[2], int (&id_new)[2])
      __attribute__((always_inline)) {
    load_ids(dense_c, c + 5, id_new);
    fetch(c + 3, id_far, far);
    PI_ISSUE_FENCE();
    convert(cur, c);
    PI_ISSUE_FENCE();
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < BD_CH / 16; ++ks) {
      const int kb = 16 * ks + 8 * (lane / 32);
      const int at = bdq_slot(BM * w + (lane & 31), kb);
      const h8v ah = *reinterpret_cast<const h8v*>(&as[0][ks][8 * lane]);
      const h8v al = *reinterpret_cast<const h8v*>(&as[1][ks][8 * lane]);
      const h8v bw = *reinterpret_cast<const h8v*>(&wt[0][at]);
      const h8v bl = *reinterpret_cast<const h8v*>(&wt[1][at]);
      acc = mfma(ah, bw, acc);
      acc = mfma(al, bw, acc);
      acc = mfma(ah, bl, acc);
    }
    __syncthreads();
    PI_ISSUE_FENCE();   // no operand math of the next chunk above the barrier (it would wait for its loads)
  };
  auto run = [&](auto dc) __attribute__((always_inline)) {
    // chunk k's row ids in slot k % 4, its loads in stage k % 4
    int id0[2], id1[2], id2[2], id3[2];
    Stage s0, s1, s2, s3;
    load_ids(dc, 0, id0);
    load_ids(dc, 1, id1);
    load_ids(dc, 2, id2);
    load_ids(dc, 3, id3);
    fetch(0, id0, s0);
    load_ids(dc, 4, id0);
    fetch(1, id1, s1);
    fetch(2, id2, s2);
    int c = 0;
    for (; c + 4 <= nch; c += 4) {
      step(dc, c, s0, s3, id3, id1);
      step(dc, c + 1, s1, s0, id0, id2);
      step(dc, c + 2, s2, s1, id1, id3);
      step(dc, c + 3, s3, s2, id2, id0);
    }
    // the last 1..3 chunks without a whole group of four (the stages are in their
    // group-start roles here)
    const int rem = nch - c;
    if (rem == 1) {
      step(dc, c, s0, s3, id3, id1);
    } else if (rem == 2) {
      step(dc, c, s0, s3, id3, id1);
      step(dc, c + 1, s1, s0, id0, id2);
    } else if (rem == 3) {
      step(dc, c, s0, s3, id3, id1);
      step(dc, c + 1, s1, s0, id0, id2);
      step(dc, c + 2, s2, s1, id1, id3);
    }
  };
  if (nch > 0) {
    if (dense)
      run(std::true_type{});
    else
      run(std::false_type{});
  }
  __syncthreads();                                 // rsc is written
  const int cg = c0 + BM * w + (lane & 31);
  if (cg < d) {
    const float bd = (b_down && split == 0) ? b_down[cg] : 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int b = 8 * g + 4 * (lane / 32) + v;
        if (b < batch) y_part[((size_t)split * BM + b) * d + cg] = acc[4 * g + v] * rsc[b] + bd;
      }
  }
}

// ------------------------------------------------- down projection (fp16)
// k_bdown's blocks, splits and chunks for fp16 weights with the pipeline of
// k_bdown_q4: thread t takes the 16-byte piece t % 32 (8 columns) of the
// block's 512-byte row segment at chunk positions 2 p and 2 p + 1 for the four
// position pairs p = t / 32 + 16 k, so 32 lanes read a row's whole segment (four
// lines) per load.  A column's positions are stored in 16-byte groups with
// group g at g ^ (c / 16 % 16): a write of the 64 lanes hits each bank at most
// twice, the MFMA reads once.  Three chunks are in flight while one is
// converted and multiplied, the row ids two steps ahead of their weights.
__host__ __device__ constexpr int bdh_slot(int col, int pos) {   // halves offset of (col, pos) in wt
  return col * BD_PAD + 8 * ((pos / 8) ^ ((col / 16) % 16)) + pos % 8;
}

__global__ void __launch_bounds__(512)
k_bdown_f16(const uint16_t* __restrict__ downT, int f, int d, const int32_t* __restrict__ ulist,
            const int32_t* __restrict__ ucount, const float* __restrict__ h32, const uint32_t* __restrict__ hmax,
            const float* __restrict__ b_down, int batch, float* __restrict__ y_part, int dense_min, int nsplit) {
  __shared__ __attribute__((aligned(16))) _Float16 wt[BD_COLS * BD_PAD];
  __shared__ __attribute__((aligned(16))) _Float16 as[2][BD_CH / 16][512];
  __shared__ float rsc[BM];
  static_assert(BD_CH == 128 && BD_COLS == 256, "32 pieces of 8 columns, 64 position pairs");
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int ngroup = (d + BD_COLS - 1) / BD_COLS;
  // consecutive launch indices go to the 8 XCDs in turn: each XCD takes a run of
  // consecutive (split, column group) items, so the column groups that share a
  // line of a row's block scales, and the blocks that share a split's h, meet in
  // one L2
  const int nblk = (int)gridDim.x;
  const int L = nblk % 8 == 0 ? (int)(blockIdx.x % 8) * (nblk / 8) + (int)blockIdx.x / 8 : (int)blockIdx.x;
  const int c0 = (L % ngroup) * BD_COLS, split = L / ngroup;
  bool dense;
  const int n = ffn_rows(ucount, f, dense_min, &dense);
  const int nch_all = (n + BD_CH - 1) / BD_CH, cps = (nch_all + nsplit - 1) / nsplit;
  const int ch0 = split * cps;
  const int nch = max(0, min(nch_all, ch0 + cps) - ch0);
  const float hs = pow2_scale(__uint_as_float(hmax[lane & 31]));
  if (tid < BM) rsc[tid] = 1.f / pow2_scale(__uint_as_float(hmax[tid]));
  // this thread's 8 columns (clamped into the row when past d, then dropped) and
  // its first position pair
  const int pc = tid & 31, rp0 = tid >> 5;
  const bool okc = c0 + 8 * pc < d;
  const int colc = min(c0 + 8 * pc, d - 8);
  f16v acc = {};

  struct Stage {
    uint4 wv[4][2];   // the 16-byte piece of the rows at positions 2 p, 2 p + 1 (p = rp0 + 16 k)
    float4 hv[2];     // 8 values of h for the A operands
  };
  // chunk c's rows (positions clamped into the list and the split); the dense and
  // the list case are separate instantiations (see k_bdown_q4)
  auto load_ids = [&](auto dense_c, int c, int (&id)[4][2]) __attribute__((always_inline)) {
    const int base = (ch0 + min(c, nch - 1)) * BD_CH + 2 * rp0;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int p = max(0, min(base + 32 * k + q, n - 1));
        id[k][q] = decltype(dense_c)::value ? p : ulist[p];
      }
  };
  auto fetch = [&](int c, const int (&id)[4][2], Stage& st) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int q = 0; q < 2; ++q)
        st.wv[k][q] = *reinterpret_cast<const uint4*>(downT + (size_t)id[k][q] * d + colc);
    const float4* hp =
        reinterpret_cast<const float4*>(h32 + (size_t)((ch0 + min(c, nch - 1)) * (BD_CH / 16) + w) * 512 + 8 * lane);
    st.hv[0] = hp[0];
    st.hv[1] = hp[1];
  };
  // a chunk's operands into LDS; positions past the split or the list and columns
  // past d are zero (h there is whatever an earlier call left)
  auto convert = [&](const Stage& st, int c) __attribute__((always_inline)) {
    const int base = (ch0 + c) * BD_CH;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int p2 = 2 * (rp0 + 16 * k);
      // zeroed by an AND with a mask (a select becomes a branch next to the loads)
      const uint32_t m0 = 0u - (uint32_t)(okc && c < nch && base + p2 < n);
      const uint32_t m1 = 0u - (uint32_t)(okc && c < nch && base + p2 + 1 < n);
      const uint32_t a[4] = {st.wv[k][0].x & m0, st.wv[k][0].y & m0, st.wv[k][0].z & m0, st.wv[k][0].w & m0};
      const uint32_t b[4] = {st.wv[k][1].x & m1, st.wv[k][1].y & m1, st.wv[k][1].z & m1, st.wv[k][1].w & m1};
      _Float16* dst = &wt[bdh_slot(8 * pc, p2)];   // the 8 columns share the swizzle
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // columns 2 j and 2 j + 1: (row p2, row p2 + 1) pairs
        *reinterpret_cast<uint32_t*>(dst + (2 * j) * BD_PAD) = __builtin_amdgcn_perm(b[j], a[j], 0x05040100u);
        *reinterpret_cast<uint32_t*>(dst + (2 * j + 1) * BD_PAD) = __builtin_amdgcn_perm(b[j], a[j], 0x07060302u);
      }
    }
    // A operands: K step w of the chunk, operand slot lane (batch row lane % 32)
    const int jj = base + 16 * w + 8 * (lane / 32);
    const float hv8[8] = {st.hv[0].x, st.hv[0].y, st.hv[0].z, st.hv[0].w,
                          st.hv[1].x, st.hv[1].y, st.hv[1].z, st.hv[1].w};
    h8v ahi, alo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      _Float16 hi, lo;
      split_f16(c < nch && jj + e < n ? hv8[e] * hs : 0.f, &hi, &lo);
      ahi[e] = hi;
      alo[e] = lo;
    }
    *reinterpret_cast<h8v*>(&as[0][w][8 * lane]) = ahi;
    *reinterpret_cast<h8v*>(&as[1][w][8 * lane]) = alo;
  };
  auto step = [&](auto dense_c, int c, const Stage& cur, Stage& far, const int (&id_far)[4][2],
                  int (&id_new)[4][2]) __attribute__((always_inline)) {
    load_ids(dense_c, c + 5, id_new);
    fetch(c + 3, id_far, far);
    PI_ISSUE_FENCE();
    convert(cur, c);
    PI_ISSUE_FENCE();
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < BD_CH / 16; ++ks) {
      const int kb = 16 * ks + 8 * (lane / 32);
      const h8v ah = *reinterpret_cast<const h8v*>(&as[0][ks][8 * lane]);
      const h8v al = *reinterpret_cast<const h8v*>(&as[1][ks][8 * lane]);
      const h8v bw = *reinterpret_cast<const h8v*>(&wt[bdh_slot(BM * w + (lane & 31), kb)]);
      acc = mfma(ah, bw, acc);
      acc = mfma(al, bw, acc);
    }
    __syncthreads();
    PI_ISSUE_FENCE();
  };
  auto run = [&](auto dc) __attribute__((always_inline)) {
    int id0[4][2], id1[4][2], id2[4][2], id3[4][2];
    Stage s0, s1, s2, s3;
    load_ids(dc, 0, id0);
    load_ids(dc, 1, id1);
    load_ids(dc, 2, id2);
    load_ids(dc, 3, id3);
    fetch(0, id0, s0);
    load_ids(dc, 4, id0);
    fetch(1, id1, s1);
    fetch(2, id2, s2);
    int c = 0;
    for (; c + 4 <= nch; c += 4) {
      step(dc, c, s0, s3, id3, id1);
      step(dc, c + 1, s1, s0, id0, id2);
      step(dc, c + 2, s2, s1, id1, id3);
      step(dc, c + 3, s3, s2, id2, id0);
    }
    // the last 1..3 chunks without a whole group of four (the stages are in their
    // group-start roles here)
    const int rem = nch - c;
    if (rem == 1) {
      step(dc, c, s0, s3, id3, id1);
    } else if (rem == 2) {
      step(dc, c, s0, s3, id3, id1);
      step(dc, c + 1, s1, s0, id0, id2);
    } else if (rem == 3) {
      step(dc, c, s0, s3, id3, id1);
      step(dc, c + 1, s1, s0, id0, id2);
      step(dc, c + 2, s2, s1, id1, id3);
    }
  };
  if (nch > 0) {
    if (dense)
      run(std::true_type{});
    else
      run(std::false_type{});
  }
  __syncthreads();                                 // rsc is written
  const int cg = c0 + BM * w + (lane & 31);
  if (cg < d) {
    const float bd = (b_down && split == 0) ? b_down[cg] : 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int b = 8 * g + 4 * (lane / 32) + v;
        if (b < batch) y_part[((size_t)split * BM + b) * d + cg] = acc[4 * g + v] * rsc[b] + bd;
      }
  }
}

// y[b] = the np partial vectors of k_bdown added in order (b < batch)
__global__ void k_bsum_y(const float* __restrict__ y_part, int np, int batch, int d, float* __restrict__ y) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= batch * d) return;
  float v = y_part[e];
  for (int p = 1; p < np; ++p) v += y_part[(size_t)p * BM * d + e];
  y[e] = v;
}

// Explicit-list input of the batched FFN: u[i] = 1 for listed i and m_nm[i][b]
// = mask[b][i] for b < batch; k_bclear first clears u and every row of m_nm
// (a dense run reads the mask bytes of every neuron).
__global__ void k_bclear(uint8_t* __restrict__ u, uint8_t* __restrict__ m_nm, int f) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < f) {
    u[i] = 0;
    uint4* m = reinterpret_cast<uint4*>(m_nm + (size_t)i * BM);
    m[0] = make_uint4(0, 0, 0, 0);
    m[1] = make_uint4(0, 0, 0, 0);
  }
}
__global__ void k_blist(const int32_t* __restrict__ idx, const int32_t* __restrict__ count, int f,
                        const uint8_t* __restrict__ mask, int batch, uint8_t* __restrict__ u,
                        uint8_t* __restrict__ m_nm) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  const int cnt = min(max(*count, 0), f);
  if (j >= cnt) return;
  const int i = idx[j];
  if (i < 0 || i >= f) return;
  u[i] = 1;
  for (int b = 0; b < BM; ++b) m_nm[(size_t)i * BM + b] = (b < batch && mask[(size_t)b * f + i]) ? 1 : 0;
}

// out[b] = glue(x[b], sum of the np partials y[p][b]) for b < batch (one
// 1024-thread block per sequence, d <= 16384); partial p of row b is at
// y_part + (p * 32 + b) * d.  Each thread's values and all their partials
// (np <= BD_MAXSPLIT) are loaded before the first add; out needs no alignment.
__global__ void __launch_bounds__(BG_T)
k_bglue_out(const float* __restrict__ x, const float* __restrict__ y_part, int np, int d, float* __restrict__ out) {
  constexpr int NJ = 16;                   // values per thread (d <= 16384)
  __shared__ float red[BG_T / WAVE];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  float v[NJ];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int k = min(tid + BG_T * j, d - 1);
    float yp[BD_MAXSPLIT];
#pragma unroll
    for (int p = 0; p < BD_MAXSPLIT; ++p) yp[p] = y_part[((size_t)min(p, np - 1) * BM + b) * d + k];
    float yv = yp[0];
#pragma unroll
    for (int p = 1; p < BD_MAXSPLIT; ++p) yv += p < np ? yp[p] : 0.f;
    v[j] = x[(size_t)b * d + k] + yv;
    if (tid + BG_T * j < d) ss = fmaf(v[j], v[j], ss);
  }
  ss = wave_sum(ss);
  if (lane == 0) red[w] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < BG_T / WAVE; ++i) tot += red[i];
  const float inv = 1.0f / sqrtf(tot / (float)d + 1e-6f);
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    if (tid + BG_T * j < d) out[(size_t)b * d + tid + BG_T * j] = v[j] * inv;
}

}  // namespace pib
