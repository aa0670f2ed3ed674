// Device code of the predictor-guided, neuron-aware sparse FFN for gfx950 (MI355X).
//
// Execution model (batch 1): one HIP stream, three kernels per layer, no
// inter-block waiting anywhere (a grid-wide barrier on this GPU costs an order
// of magnitude more than a kernel boundary in a HIP graph):
//   K1 k_predict_t  residual RMS glue (recomputed identically by every block)
//                   and the predictor's first GEMV t = A x
//   K2 k_score      predictor second GEMV s = B t + b, threshold s > 0, mask
//                   bits, and -- fused -- the gathered up/gate GEMV with ReLU or
//                   ReGLU for the block's active neurons (h per neuron)
//   K3 k_down       down projection over active neurons, tiled by column tile x
//                   neuron sub-chunk; each wave walks its neurons in ascending
//                   order (ballot over the mask bits), the block reduces its
//                   waves in a fixed order and adds one fp64 value per column
//
// Loads are 16 bytes per lane (4 fp32, 8 fp16 or one Q4_0 block of 32 nibbles)
// so that a wave reads 1 KiB contiguous per instruction; vectors that every
// row meets (x, t) are staged in LDS.  Cross-lane sums are butterflies, so
// every lane ends with the same bits and decisions are wave-uniform.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pik {

enum { DT_F32 = 0, DT_F16 = 1, DT_Q4 = 2 };
enum { ACT_RELU = 0, ACT_REGLU = 1 };

constexpr int WAVE = 64;

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

template <int DT> struct Tr;
template <> struct Tr<DT_F32> { static constexpr int EPL = 4; };   // elements per 16-byte chunk
template <> struct Tr<DT_F16> { static constexpr int EPL = 8; };
template <> struct Tr<DT_Q4>  { static constexpr int EPL = 32; };

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, WAVE);
  return v;
}

// 16-byte chunk of row `row` starting at element `e` (a multiple of EPL).
template <int DT>
__device__ __forceinline__ uint4 ld_chunk(const void* __restrict__ w, size_t row, int n, int e) {
  if constexpr (DT == DT_F32) {
    return *reinterpret_cast<const uint4*>(static_cast<const float*>(w) + row * (size_t)n + e);
  } else if constexpr (DT == DT_F16) {
    return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(w) + row * (size_t)n + e);
  } else {
    return *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(w) + row * (size_t)(n / 2) + e / 2);
  }
}

// Q4_0 block scale of the block that starts at element e.
__device__ __forceinline__ float ld_scale(const uint16_t* __restrict__ sc, size_t row, int n, int e) {
  const uint16_t b = sc[row * (size_t)(n / 32) + e / 32];
  return (float)__builtin_bit_cast(_Float16, b);
}

// sum_j w_j * x_j over one chunk; x points at LDS (element e of the vector).
template <int DT>
__device__ __forceinline__ float chunk_dot(uint4 c, float scale, const float* __restrict__ x) {
  if constexpr (DT == DT_F32) {
    const float4 xv = *reinterpret_cast<const float4*>(x);
    float a = __uint_as_float(c.x) * xv.x;
    a = fmaf(__uint_as_float(c.y), xv.y, a);
    a = fmaf(__uint_as_float(c.z), xv.z, a);
    a = fmaf(__uint_as_float(c.w), xv.w, a);
    return a;
  } else if constexpr (DT == DT_F16) {
    const half8_t h = __builtin_bit_cast(half8_t, c);
    const float4 x0 = *reinterpret_cast<const float4*>(x);
    const float4 x1 = *reinterpret_cast<const float4*>(x + 4);
    float a = (float)h[0] * x0.x;
    a = fmaf((float)h[1], x0.y, a);
    a = fmaf((float)h[2], x0.z, a);
    a = fmaf((float)h[3], x0.w, a);
    a = fmaf((float)h[4], x1.x, a);
    a = fmaf((float)h[5], x1.y, a);
    a = fmaf((float)h[6], x1.z, a);
    a = fmaf((float)h[7], x1.w, a);
    return a;
  } else {
    // weight j < 16: low nibble of byte j; weight j + 16: high nibble of byte j
    const uint32_t wd[4] = {c.x, c.y, c.z, c.w};
    float a = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t byte = (wd[k] >> (8 * b)) & 0xFFu;
        const int j = 4 * k + b;
        a = fmaf((float)((int)(byte & 15u) - 8), x[j], a);
        a = fmaf((float)((int)(byte >> 4) - 8), x[j + 16], a);
      }
    }
    return a * scale;
  }
}

// acc[j] += h * w_j over one chunk (acc has EPL entries).
template <int DT>
__device__ __forceinline__ void chunk_axpy(uint4 c, float scale, float h, float* __restrict__ acc) {
  if constexpr (DT == DT_F32) {
    acc[0] = fmaf(h, __uint_as_float(c.x), acc[0]);
    acc[1] = fmaf(h, __uint_as_float(c.y), acc[1]);
    acc[2] = fmaf(h, __uint_as_float(c.z), acc[2]);
    acc[3] = fmaf(h, __uint_as_float(c.w), acc[3]);
  } else if constexpr (DT == DT_F16) {
    const half8_t v = __builtin_bit_cast(half8_t, c);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = fmaf(h, (float)v[j], acc[j]);
  } else {
    const float hs = h * scale;
    const uint32_t wd[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t byte = (wd[k] >> (8 * b)) & 0xFFu;
        const int j = 4 * k + b;
        acc[j] = fmaf(hs, (float)((int)(byte & 15u) - 8), acc[j]);
        acc[j + 16] = fmaf(hs, (float)((int)(byte >> 4) - 8), acc[j + 16]);
      }
    }
  }
}

// Row `row` of a [rows][n] matrix dotted with the LDS vector xs[n]; full wave sum.
template <int DT>
__device__ __forceinline__ float row_dot(const void* __restrict__ w, const uint16_t* __restrict__ sc,
                                         size_t row, int n, const float* __restrict__ xs, int lane) {
  constexpr int EPL = Tr<DT>::EPL;
  float a = 0.f;
#pragma unroll 4
  for (int e = lane * EPL; e < n; e += WAVE * EPL) {
    const uint4 c = ld_chunk<DT>(w, row, n, e);
    const float s = (DT == DT_Q4) ? ld_scale(sc, row, n, e) : 1.f;
    a += chunk_dot<DT>(c, s, xs + e);
  }
  return wave_sum(a);
}

// ----------------------------------------------------------------------- K1
// t = A x', x' = glue(x_prev, y_prev) if y_prev != NULL else x_prev.
// glue: v = x_prev + y_prev; x' = v / sqrt(mean(v^2) + 1e-6).  Every block
// computes the same x' with the same operation order, so all blocks agree
// bit for bit.  Blocks also write their slice of x' and clear their slice of
// the next layer's accumulators.
template <int PT>
__global__ void __launch_bounds__(256)
k_predict_t(const void* __restrict__ A, int r, int d, const float* __restrict__ x_prev,
            const double* __restrict__ y_prev, float* __restrict__ x_out, float* __restrict__ x_trace,
            float* __restrict__ t, double* __restrict__ zero_y, int zero_y_n,
            uint32_t* __restrict__ zero_w, int zero_w_n) {
  extern __shared__ float xs[];
  __shared__ float red[16];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE, W = blockDim.x / WAVE;

  float ss = 0.f;
  for (int k = tid; k < d; k += blockDim.x) {
    float v = x_prev[k];
    if (y_prev) v += (float)y_prev[k];
    xs[k] = v;
    ss = fmaf(v, v, ss);
  }
  if (y_prev) {
    ss = wave_sum(ss);
    if (lane == 0) red[w] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int i = 0; i < W; ++i) tot += red[i];
    const float inv = 1.0f / sqrtf(tot / (float)d + 1e-6f);
    for (int k = tid; k < d; k += blockDim.x) xs[k] *= inv;
  }
  __syncthreads();

  // slices: x' out, trace, zeroing
  {
    const int nb = gridDim.x, b = blockIdx.x;
    const int cx = (d + nb - 1) / nb;
    for (int k = b * cx + tid; k < min(d, (b + 1) * cx); k += blockDim.x) {
      if (x_out) x_out[k] = xs[k];
      if (x_trace) x_trace[k] = xs[k];
    }
    if (zero_y) {
      const int cy = (zero_y_n + nb - 1) / nb;
      for (int k = b * cy + tid; k < min(zero_y_n, (b + 1) * cy); k += blockDim.x) zero_y[k] = 0.0;
    }
    if (zero_w) {
      const int cw = (zero_w_n + nb - 1) / nb;
      for (int k = b * cw + tid; k < min(zero_w_n, (b + 1) * cw); k += blockDim.x) zero_w[k] = 0u;
    }
  }

  for (int j = blockIdx.x * W + w; j < r; j += gridDim.x * W) {
    const float a = row_dot<PT>(A, nullptr, (size_t)j, d, xs, lane);
    if (lane == 0) t[j] = a;
  }
}

// ----------------------------------------------------------------------- K2
// Block b owns neurons i = b + gridDim.x * m (interleaved, so that hot-first
// order does not load the first blocks more than the last).  Scores for all
// of them, then -- if FUSE_UP -- the up/gate dot products of the active ones.
constexpr int K2_MAX_PER_BLOCK = 256;

template <int PT, int WT, int ACT, bool FUSE_UP>
__global__ void __launch_bounds__(256)
k_score(const void* __restrict__ Bm, const float* __restrict__ pbias, const float* __restrict__ bias,
        const float* __restrict__ t, int f, int r,
        const void* __restrict__ gate_w, const uint16_t* __restrict__ gate_sc,
        const void* __restrict__ up_w, const uint16_t* __restrict__ up_sc,
        const float* __restrict__ xcur, int d,
        float* __restrict__ scores, uint8_t* __restrict__ mask_u8,
        uint32_t* __restrict__ mask_bits, float* __restrict__ h_full) {
  extern __shared__ float smem[];
  float* ts = smem;        // [r]
  float* xs = smem + r;    // [d] (FUSE_UP only)
  __shared__ int act_list[K2_MAX_PER_BLOCK];
  __shared__ int n_act;
  constexpr int PEPL = Tr<PT>::EPL;
  constexpr int U = 4;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE, W = blockDim.x / WAVE;
  const int NB = gridDim.x, b = blockIdx.x;

  for (int k = tid; k < r; k += blockDim.x) ts[k] = t[k];
  if (tid == 0) n_act = 0;
  __syncthreads();

  const int M = (f - b + NB - 1) / NB;   // neurons of this block (b < f)
  for (int m0 = w; m0 < M; m0 += W * U) {
    float acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = 0.f;
    for (int e = lane * PEPL; e < r; e += WAVE * PEPL) {
      uint4 c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int m = m0 + u * W;
        if (m < M) c[u] = ld_chunk<PT>(Bm, (size_t)b + (size_t)NB * m, r, e);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int m = m0 + u * W;
        if (m < M) acc[u] += chunk_dot<PT>(c[u], 1.f, ts + e);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int m = m0 + u * W;
      if (m < M) {
        const int i = b + NB * m;
        const float s = wave_sum(acc[u]) + pbias[i];
        const bool on = s > 0.f;
        if (lane == 0) {
          if (scores) scores[i] = s;
          if (mask_u8) mask_u8[i] = on ? 1 : 0;
          if (on) {
            atomicOr(&mask_bits[i >> 5], 1u << (i & 31));
            if constexpr (FUSE_UP) act_list[atomicAdd(&n_act, 1)] = i;
          }
        }
      }
    }
  }
  if constexpr (FUSE_UP) {
    __syncthreads();
    const int na = n_act;
    if (na == 0) return;
    for (int k = tid; k < d; k += blockDim.x) xs[k] = xcur[k];
    __syncthreads();
    for (int a = w; a < na; a += W) {
      const int i = act_list[a];
      const float zu = row_dot<WT>(up_w, up_sc, (size_t)i, d, xs, lane);
      float h;
      if constexpr (ACT == ACT_RELU) {
        h = fmaxf(zu + bias[i], 0.f);
      } else {
        const float zg = row_dot<WT>(gate_w, gate_sc, (size_t)i, d, xs, lane);
        h = fmaxf(zg + bias[i], 0.f) * zu;
      }
      if (lane == 0) h_full[i] = h;
    }
  }
}

// Up/gate over an explicit list (pi_sparse_ffn): h_list[j] for j < count.
// Block 0's threads also clear the fp64 accumulator y_acc[d].
template <int WT, int ACT>
__global__ void __launch_bounds__(256)
k_up_list(const void* __restrict__ gate_w, const uint16_t* __restrict__ gate_sc,
          const void* __restrict__ up_w, const uint16_t* __restrict__ up_sc,
          const float* __restrict__ bias, const float* __restrict__ x, int d, int f,
          const int32_t* __restrict__ idx, const int32_t* __restrict__ count,
          float* __restrict__ h_list, double* __restrict__ y_acc) {
  extern __shared__ float xs[];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE, W = blockDim.x / WAVE;
  {
    const int nb = gridDim.x, b = blockIdx.x, cy = (d + nb - 1) / nb;
    for (int k = b * cy + tid; k < min(d, (b + 1) * cy); k += blockDim.x) y_acc[k] = 0.0;
  }
  const int cnt = min(max(*count, 0), f);
  if ((int)blockIdx.x * W >= cnt) return;
  for (int k = tid; k < d; k += blockDim.x) xs[k] = x[k];
  __syncthreads();
  for (int j = blockIdx.x * W + w; j < cnt; j += gridDim.x * W) {
    const int i = idx[j];
    float h = 0.f;
    if (i >= 0 && i < f) {
      const float zu = row_dot<WT>(up_w, up_sc, (size_t)i, d, xs, lane);
      if constexpr (ACT == ACT_RELU) {
        h = fmaxf(zu + bias[i], 0.f);
      } else {
        const float zg = row_dot<WT>(gate_w, gate_sc, (size_t)i, d, xs, lane);
        h = fmaxf(zg + bias[i], 0.f) * zu;
      }
    }
    if (lane == 0) h_list[j] = h;
  }
}

// ----------------------------------------------------------------------- K3
// Down projection.  Block (ct, nc): column tile ct of width 64*EPL, neuron
// sub-chunks s = nc*W + w (of S = NC*W).  Wave s accumulates, in ascending
// neuron order, the active neurons i with i % S == s (implicit mode: mask
// bits + h per neuron) or the list positions j % S == s (explicit mode: idx +
// h per position).  Block partials are summed over waves in a fixed order
// and added to y_acc (fp64) with one atomic per column.
template <int WT, bool EXPLICIT>
__global__ void __launch_bounds__(256)
k_down(const void* __restrict__ downT, const uint16_t* __restrict__ down_sc, int f, int d, int CT,
       const uint32_t* __restrict__ mask_bits, const float* __restrict__ h_full,
       const int32_t* __restrict__ idx, const int32_t* __restrict__ count, const float* __restrict__ h_list,
       const float* __restrict__ b_down, double* __restrict__ y_acc, int32_t* __restrict__ count_out) {
  constexpr int EPL = Tr<WT>::EPL;
  constexpr int TW = WAVE * EPL;
  constexpr int U = 4;
  extern __shared__ float red[];   // [W][TW]
  __shared__ int cnt_red[16];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE, W = blockDim.x / WAVE;
  const int ct = blockIdx.x % CT, nc = blockIdx.x / CT, NC = gridDim.x / CT;
  const int S = NC * W, s = nc * W + w;
  const int col = ct * TW + lane * EPL;
  const bool col_ok = col < d;

  if (!EXPLICIT && count_out && blockIdx.x == 0) {
    int c = 0;
    const int nwords = (f + 31) / 32;
    for (int k = tid; k < nwords; k += blockDim.x) c += __popc(mask_bits[k]);
    for (int m = 32; m >= 1; m >>= 1) c += __shfl_xor(c, m, WAVE);
    if (lane == 0) cnt_red[w] = c;
    __syncthreads();
    if (tid == 0) {
      int tot = 0;
      for (int i = 0; i < W; ++i) tot += cnt_red[i];
      *count_out = tot;
    }
  }

  float acc[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) acc[j] = 0.f;

  const int n_items = EXPLICIT ? min(max(*count, 0), f) : f;
  for (int base = s; base < n_items; base += S * WAVE) {
    const int item = base + S * lane;
    bool on = false;
    if (item < n_items) {
      if constexpr (EXPLICIT) {
        const int i = idx[item];
        on = (i >= 0) && (i < f);
      } else {
        on = (mask_bits[item >> 5] >> (item & 31)) & 1u;
      }
    }
    uint64_t bal = __ballot(on);
    while (bal) {
      int rows[U];
      float hv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        rows[u] = -1;
        hv[u] = 0.f;
        if (bal) {
          const int l = __ffsll((unsigned long long)bal) - 1;
          bal &= bal - 1;
          const int it = base + S * l;
          if constexpr (EXPLICIT) {
            rows[u] = idx[it];
            hv[u] = h_list[it];
          } else {
            rows[u] = it;
            hv[u] = h_full[it];
          }
        }
      }
      uint4 c[U];
      float sc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        sc[u] = 1.f;
        if (rows[u] >= 0 && col_ok) {
          c[u] = ld_chunk<WT>(downT, (size_t)rows[u], d, col);
          if constexpr (WT == DT_Q4) sc[u] = ld_scale(down_sc, (size_t)rows[u], d, col);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (rows[u] >= 0 && col_ok) chunk_axpy<WT>(c[u], sc[u], hv[u], acc);
    }
  }

#pragma unroll
  for (int j = 0; j < EPL; ++j) red[w * TW + lane * EPL + j] = acc[j];
  __syncthreads();
  for (int cc = tid; cc < TW; cc += blockDim.x) {
    const int cg = ct * TW + cc;
    if (cg >= d) continue;
    float v = 0.f;
    for (int i = 0; i < W; ++i) v += red[i * TW + cc];
    if (b_down && nc == 0) v += b_down[cg];
    unsafeAtomicAdd(&y_acc[cg], (double)v);
  }
}

// --------------------------------------------------------------- small ones
// Ascending list of set mask bits (single block): idx[0..count), *count.
__global__ void __launch_bounds__(1024)
k_compact(const uint32_t* __restrict__ mask_bits, int f, int32_t* __restrict__ idx, int32_t* __restrict__ count) {
  __shared__ int wsum[16];
  __shared__ int base_s;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE, W = blockDim.x / WAVE;
  const int nwords = (f + 31) / 32;
  if (tid == 0) base_s = 0;
  __syncthreads();
  for (int w0 = 0; w0 < nwords; w0 += blockDim.x) {
    const int k = w0 + tid;
    const uint32_t bits = k < nwords ? mask_bits[k] : 0u;
    const int c = __popc(bits);
    // inclusive scan within the wave
    int inc = c;
    for (int off = 1; off < WAVE; off <<= 1) {
      const int v = __shfl_up(inc, off, WAVE);
      if (lane >= off) inc += v;
    }
    if (lane == WAVE - 1) wsum[w] = inc;
    __syncthreads();
    int wbase = 0;
    for (int i = 0; i < w; ++i) wbase += wsum[i];
    const int pos = base_s + wbase + inc - c;
    uint32_t bb = bits;
    int o = 0;
    while (bb) {
      const int bit = __ffs(bb) - 1;
      bb &= bb - 1;
      idx[pos + o++] = k * 32 + bit;
    }
    __syncthreads();
    if (tid == 0) {
      int tot = 0;
      for (int i = 0; i < W; ++i) tot += wsum[i];
      base_s += tot;
    }
    __syncthreads();
  }
  if (tid == 0) *count = base_s;
}

__global__ void k_copy_i32(const int32_t* __restrict__ src, int32_t* __restrict__ dst, int n) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k < n) dst[k] = src[k];
}

// y = float(y_acc)
__global__ void k_finalize(const double* __restrict__ y_acc, float* __restrict__ y, int n) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k < n) y[k] = (float)y_acc[k];
}

// out = glue(x, y_acc): single block, same operation order as K1's glue.
__global__ void __launch_bounds__(256)
k_glue_out(const float* __restrict__ x, const double* __restrict__ y_acc, float* __restrict__ out, int d) {
  extern __shared__ float vs[];
  __shared__ float red[16];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE, W = blockDim.x / WAVE;
  float ss = 0.f;
  for (int k = tid; k < d; k += blockDim.x) {
    const float v = x[k] + (float)y_acc[k];
    vs[k] = v;
    ss = fmaf(v, v, ss);
  }
  ss = wave_sum(ss);
  if (lane == 0) red[w] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int i = 0; i < W; ++i) tot += red[i];
  const float inv = 1.0f / sqrtf(tot / (float)d + 1e-6f);
  for (int k = tid; k < d; k += blockDim.x) out[k] = vs[k] * inv;
}

}  // namespace pik
