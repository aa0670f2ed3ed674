// Device code of the predictor-guided, neuron-aware sparse FFN for gfx950 (MI355X).
//
// Execution model (batch 1): one HIP stream, three kernels per layer, no
// inter-block waiting and no global atomics anywhere (on this GPU a grid-wide
// barrier costs far more than a kernel boundary in a HIP graph, and a kernel
// that issues device-scope atomics pays their full round trip before it can
// retire):
//   K1 k_predict_t  residual RMS glue (recomputed identically by every block)
//                   and the predictor's first GEMV t = A x
//   K2 k_score      predictor second GEMV s = B t + c and threshold s > 0 for
//                   every neuron, then -- fused -- the gathered up/gate GEMV
//                   with its activation for the block's active neurons, all of
//                   the block's lanes on each row; per-block lists of the
//                   (neuron, h) pairs with h != 0
//   K3 k_down       down projection over the listed neurons; each block owns a
//                   column tile (and one of NC neuron splits), copies its share
//                   of the lists into LDS, gathers their row segments and
//                   writes its partial y with plain stores; the consumer adds
//                   the NC partials in a fixed order
//
// Weight loads are 16 bytes per lane (4 fp32, 8 fp16 or one Q4_0 block of 32
// nibbles).  Every batch of loads is issued unconditionally (indices clamped
// to valid addresses, surplus results masked) and fenced from its uses, so a
// wave has a whole batch in flight per HBM round trip.  Cross-lane sums are
// butterflies in a fixed order, so results are bit-reproducible.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace pik {

enum { DT_F32 = 0, DT_F16 = 1, DT_Q4 = 2 };
enum { ACT_RELU = 0, ACT_REGLU = 1, ACT_RELU2 = 2 };

// Matrices an activation reads per neuron: the gate and up rows for ReGLU,
// the up row alone for ReLU and Squared ReLU.
template <int ACT> constexpr int act_nmat() { return ACT == ACT_REGLU ? 2 : 1; }

// h from the gate (ReGLU) or up (ReLU, Squared ReLU) dot product zg, its bias
// b and, for ReGLU, the up dot product zu:
//   ReLU max(zg + b, 0); ReGLU max(zg + b, 0) * zu; Squared ReLU max(zg + b, 0)^2.
template <int ACT>
__device__ __forceinline__ float act_h(float zg, float b, float zu) {
  const float r = fmaxf(zg + b, 0.f);
  if constexpr (ACT == ACT_REGLU) return r * zu;
  else if constexpr (ACT == ACT_RELU2) return r * r;
  else return r;
}

constexpr int WAVE = 64;

// Keeps the instruction scheduler from moving instructions across this point.
// Placed after a batch of loads so that the whole batch is issued before the
// first use of any of it: left alone, the scheduler interleaves load, wait and
// use to save registers, which turns one memory round trip into many.
#define PI_ISSUE_FENCE() __builtin_amdgcn_sched_barrier(0)

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

template <int DT> struct Tr;
template <> struct Tr<DT_F32> { static constexpr int EPL = 4; };   // elements per 16-byte chunk
template <> struct Tr<DT_F16> { static constexpr int EPL = 8; };
template <> struct Tr<DT_Q4>  { static constexpr int EPL = 32; };

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

// Wave-uniform lane read (v_readlane): the value of `v` in lane `l`.
__device__ __forceinline__ int lane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Cross-lane moves through DPP (a VALU operand modifier, no LDS round trip).
// Lanes whose source is outside the row, and rows not in ROW_MASK, read 0.
//   0x111..0x11F  row_shr:1..15  (lane i reads lane i-n of its 16-lane row)
//   0x142         row_bcast:15   (lane 15 of each row feeds the next row)
//   0x143         row_bcast:31   (lane 31 feeds rows 2 and 3)
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, false);
}

// Inclusive prefix sum over the 64 lanes (Hillis-Steele inside each row, then
// the row totals carried across rows).  The order of additions is fixed.
__device__ __forceinline__ float wave_scan(float x) {
  x += dpp_f<0x111>(x);
  x += dpp_f<0x112>(x);
  x += dpp_f<0x114>(x);
  x += dpp_f<0x118>(x);
  x += dpp_f<0x142, 0xa>(x);
  x += dpp_f<0x143, 0xc>(x);
  return x;
}
__device__ __forceinline__ int wave_scan(int x) {
  x += dpp_i<0x111>(x);
  x += dpp_i<0x112>(x);
  x += dpp_i<0x114>(x);
  x += dpp_i<0x118>(x);
  x += dpp_i<0x142, 0xa>(x);
  x += dpp_i<0x143, 0xc>(x);
  return x;
}

// Sum over the wave, the same wave-uniform value in every lane.
__device__ __forceinline__ float wave_sum(float v) { return lane_f(wave_scan(v), WAVE - 1); }

// Maximum over the wave of non-negative values (a prefix maximum with the
// same steps as wave_scan; lanes shifted in from outside read 0), in every lane.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<0x111>(x));
  x = fmaxf(x, dpp_f<0x112>(x));
  x = fmaxf(x, dpp_f<0x114>(x));
  x = fmaxf(x, dpp_f<0x118>(x));
  x = fmaxf(x, dpp_f<0x142, 0xa>(x));
  x = fmaxf(x, dpp_f<0x143, 0xc>(x));
  return lane_f(x, WAVE - 1);
}
__device__ __forceinline__ int wave_sum(int v) { return lane_i(wave_scan(v), WAVE - 1); }

// Sum over the lanes that share lane % G (G = 1, 2, 4, 8 or 16): a scan with
// row shifts that are multiples of G inside each 16-lane row, then the four
// row totals (lanes 16 r + 16 - G + q) added in row order.  The result for
// residue q is wave-uniform; `res` holds it for q = lane % G.
template <int G>
__device__ __forceinline__ float group_sum(float x, int lane) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "bad group");
  if constexpr (G <= 1) x += dpp_f<0x111>(x);
  if constexpr (G <= 2) x += dpp_f<0x110 + 2>(x);
  if constexpr (G <= 4) x += dpp_f<0x110 + 4>(x);
  if constexpr (G <= 8) x += dpp_f<0x110 + 8>(x);
  float res = 0.f;
#pragma unroll
  for (int q = 0; q < G; ++q) {
    const float t = lane_f(x, 16 - G + q) + lane_f(x, 32 - G + q) + lane_f(x, 48 - G + q) + lane_f(x, 64 - G + q);
    if ((lane % G) == q) res = t;
  }
  return res;
}

// Sum over the lanes of each 16-lane row that share lane % G (G = 1, 2, 4, 8
// or 16), left in the row's last G lanes: lane 16 r + 16 - G + q holds the sum
// for residue q of row r.  Row shifts that are multiples of G, added in a
// fixed order; the other lanes hold partial sums.
template <int G>
__device__ __forceinline__ float row_group_sum(float x) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "bad group");
  if constexpr (G <= 1) x += dpp_f<0x111>(x);
  if constexpr (G <= 2) x += dpp_f<0x112>(x);
  if constexpr (G <= 4) x += dpp_f<0x114>(x);
  if constexpr (G <= 8) x += dpp_f<0x118>(x);
  return x;
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
    static_assert(DT != DT_Q4, "Q4_0 rows are dotted with chunk_dot_q4t");
    return 0.f;
  }
}

// A value the compiler cannot see through (an SGPR set by inline asm).  Adding
// it to the addresses of a batch of loads makes them depend on this point of
// the program, so they cannot be hoisted above it.
__device__ __forceinline__ int opaque_zero() {
  int z;
  asm volatile("s_mov_b32 %0, 0" : "=s"(z));
  return z;
}

// The low and the high nibble of each byte of w, each in a byte of its own
// (w & 0x0F0F0F0F, (w >> 4) & 0x0F0F0F0F), with a mask the compiler cannot
// see as a constant.  Seeing it, the compiler extracts every nibble with a
// bit-field instruction of its own before converting it; this way each byte
// is converted in place (v_cvt_f32_ubyte0..3): one instruction per weight.
__device__ __forceinline__ uint32_t nib_mask() { return 0x0F0F0F0Fu + (uint32_t)opaque_zero(); }
__device__ __forceinline__ float ubyte_f(uint32_t w, int b) { return (float)((w >> (8 * b)) & 0xFFu); }

// Q4_0 activations in LDS for the gathered dot products, pair-transposed:
// element 32 b + j (block b, 0 <= j < 32) is half j / 16 of the float2 at
// xq[(j % 16) * nb + b], nb = d / 32.  A lane that owns block b reads its 16
// pairs at stride nb, so the 64 lanes of a wave read 64 consecutive 8-byte
// words per access: no LDS bank conflicts (the linear layout puts the lanes
// 128 bytes apart, all on the same banks).  The block sums of x follow the d
// values: xq[d + b] = sum of the 32 elements of block b.
__host__ __device__ constexpr int q4t_pos(int k, int d) { return ((k & 15) * (d >> 5) + (k >> 5)) * 2 + ((k >> 4) & 1); }
// floats of a pair-transposed x with its block sums (padded to whole 16-byte vectors)
__host__ __device__ constexpr int q4t_len(int d) { return d + ((d >> 5) + 3) / 4 * 4; }

// sum_j w_j * x_j over Q4_0 block `blk`, x in the pair-transposed layout and
// xsum the block's sum of x: sum_j d (q_j - 8) x_j = d (sum_j q_j x_j - 8 xsum),
// so each weight costs one conversion and one FMA.
__device__ __forceinline__ float chunk_dot_q4t(uint4 c, float scale, const float2* __restrict__ xq, int blk, int nb,
                                               float xsum) {
  const uint32_t wd[4] = {c.x, c.y, c.z, c.w};
  const uint32_t m = nib_mask();
  float a = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t lo = wd[k] & m, hi = (wd[k] >> 4) & m;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float2 xv = xq[(4 * k + b) * nb + blk];
      a = fmaf(ubyte_f(lo, b), xv.x, a);
      a = fmaf(ubyte_f(hi, b), xv.y, a);
    }
  }
  return fmaf(-8.f, xsum, a) * scale;
}

// acc[j] += h * w_j over one chunk (acc has EPL entries).  For Q4_0 it adds
// h d q_j and leaves the -8 offset to the caller: hsum collects h d, and
// acc[j] - 8 hsum is the sum of h d (q_j - 8) = h w_j.
template <int DT>
__device__ __forceinline__ void chunk_axpy(uint4 c, float scale, float h, float* __restrict__ acc, float& hsum) {
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
    hsum += hs;
    const uint32_t wd[4] = {c.x, c.y, c.z, c.w};
    const uint32_t m = nib_mask();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = wd[k] & m, hi = (wd[k] >> 4) & m;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int j = 4 * k + b;
        acc[j] = fmaf(hs, ubyte_f(lo, b), acc[j]);
        acc[j + 16] = fmaf(hs, ubyte_f(hi, b), acc[j + 16]);
      }
    }
  }
}

// Copy n floats (n % 4 == 0, both pointers 16-byte aligned) from global memory
// to LDS, starting at float4 index `first`.  A thread issues all MAXV 16-byte
// loads of a round before the first store; indices past the end are clamped to
// the last vector, which is then loaded and stored twice with the same value,
// so no load sits in a branch (a load in a branch is sunk next to its use and
// the batch is lost).
template <int MAXV>
__device__ __forceinline__ void stage_f32(float* __restrict__ lds, const float* __restrict__ g, int n, int tid,
                                          int nthr, int first = 0) {
  const int nv = n / 4;
  for (int base = first; base < nv; base += MAXV * nthr) {
    float4 v[MAXV];
#pragma unroll
    for (int j = 0; j < MAXV; ++j) v[j] = reinterpret_cast<const float4*>(g)[min(base + j * nthr + tid, nv - 1)];
    PI_ISSUE_FENCE();
#pragma unroll
    for (int j = 0; j < MAXV; ++j) reinterpret_cast<float4*>(lds)[min(base + j * nthr + tid, nv - 1)] = v[j];
  }
}

// ------------------------------------------------------------- LDS-DMA

// Wait until at most N vector-memory loads of this wave are outstanding and
// all its LDS operations are done.  Loads complete in issue order, so this
// waits for everything issued before the last N.
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// LDS floats that dma_f32 writes for n floats: whole 1 KB pieces.
__host__ __device__ constexpr int dma_pad(int n) { return (n + 255) / 256 * 256; }

// Copy n floats (n % 4 == 0, g 16-byte aligned) from global memory straight
// into lds[0, dma_pad(n)) with LDS-DMA loads (global_load_lds_dwordx4): lane i
// of a wave-wide load lands at 16 i bytes past the piece's base.  Wave w of nw
// issues 1 KB pieces w, w + nw, ...; lanes past n read the last vector again
// and write the padding.  No registers hold the data, so the loads cannot be
// sunk to a later use; the data is in LDS once this wave's vmcnt has passed
// them, and visible to the other waves after a barrier that follows that wait.
__device__ __forceinline__ void dma_f32(float* lds, const float* g, int n, int w, int nw, int lane) {
  const int nv = n / 4, npc = (nv + 63) / 64;
  for (int c = w; c < npc; c += nw)
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)(g + 4 * min(c * 64 + lane, nv - 1)),
        (__attribute__((address_space(3))) void*)(lds + c * 256), 16, 0, 0);
}

// v = x + sum_{p < np} y[p] (np partial vectors of n floats, added in the
// order p = 0, 1, ...) into LDS, returning this thread's sum of v^2 over its
// elements in a fixed order.  np == 0: v = x.
__device__ __forceinline__ float stage_residual(float* __restrict__ lds, const float* __restrict__ x,
                                                const float* __restrict__ y, int np, int n, int tid, int nthr) {
  const int nv = n / 4;
  float ss = 0.f;
  for (int k = tid; k < nv; k += nthr) {
    float4 v = reinterpret_cast<const float4*>(x)[k];
    if (np > 0) {
      float4 y4 = reinterpret_cast<const float4*>(y)[k];
      for (int p = 1; p < np; ++p) {
        const float4 u = reinterpret_cast<const float4*>(y + (size_t)p * n)[k];
        y4.x += u.x;
        y4.y += u.y;
        y4.z += u.z;
        y4.w += u.w;
      }
      v.x += y4.x;
      v.y += y4.y;
      v.z += y4.z;
      v.w += y4.w;
    }
    reinterpret_cast<float4*>(lds)[k] = v;
    ss = fmaf(v.x, v.x, ss);
    ss = fmaf(v.y, v.y, ss);
    ss = fmaf(v.z, v.z, ss);
    ss = fmaf(v.w, v.w, ss);
  }
  return ss;
}

// Dot products of rows rows[0..NN) of NMAT matrices (NMAT = 2: gate, up) with
// the LDS vector xs[d] (for Q4_0 pair-transposed, with its block sums: see q4t_pos): all NN * NMAT * NCH chunk
// loads of a round are issued
// before the first multiply, one HBM round trip per round.  z[n][m] is row
// rows[n] of matrix m dotted with xs, in every lane.  Chunks past the row
// (ragged tail, or beyond the row's chunk count) load a clamped, valid address
// and are masked out of the sum.
template <int WT, int NCH, int NMAT, int NN>
__device__ __forceinline__ void gather_rows(const void* __restrict__ w0, const uint16_t* __restrict__ s0,
                                            const void* __restrict__ w1, const uint16_t* __restrict__ s1,
                                            const int (&rows)[NN], int d, const float* __restrict__ xs, int lane,
                                            float (&z)[NN][NMAT]) {
  constexpr int EPL = Tr<WT>::EPL, TW = WAVE * EPL, NV = NN * NMAT;
  const int nch = (d + TW - 1) / TW;
  float a[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) a[v] = 0.f;
  for (int q0 = 0; q0 < nch; q0 += NCH) {
    uint4 c[NV][NCH];
    float fs[NV][NCH];
#pragma unroll
    for (int n = 0; n < NN; ++n)
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int q = 0; q < NCH; ++q) {
          const int e = min(min(q0 + q, nch - 1) * TW + lane * EPL, d - EPL);
          c[n * NMAT + m][q] = ld_chunk<WT>(m ? w1 : w0, (size_t)rows[n], d, e);
          fs[n * NMAT + m][q] = (WT == DT_Q4) ? ld_scale(m ? s1 : s0, (size_t)rows[n], d, e) : 1.f;
        }
    PI_ISSUE_FENCE();
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      const int e = (q0 + q) * TW + lane * EPL;
      const bool ok = (q0 + q < nch) && (e < d);
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        float p;
        if constexpr (WT == DT_Q4)
          p = chunk_dot_q4t(c[v][q], fs[v][q], reinterpret_cast<const float2*>(xs), ok ? e / 32 : 0, d / 32,
                            xs[d + (ok ? e / 32 : 0)]);
        else
          p = chunk_dot<WT>(c[v][q], fs[v][q], xs + (ok ? e : 0));
        a[v] += ok ? p : 0.f;
      }
    }
  }
#pragma unroll
  for (int v = 0; v < NV; ++v) z[v / NMAT][v % NMAT] = wave_sum(a[v]);
}

// ----------------------------------------------------------------------- K1
// The predictor's first product in KS column slices: t_part[k][row] =
// A[row, slice k] . v[slice k].  v is the layer's input before the glue (the
// residual sum x + y that the previous layer's down projection wrote, or the
// stack's input).  The glue's normalisation x' = v / sqrt(mean(v^2) + 1e-6)
// is a scalar factor, so the score kernel applies it to the sum of the
// slices' products; with a glue, the blocks of row group 0 write their
// slice's sum of squares ss[k] for it.
// Block b takes slice k = b % KS and rows 8 (b / KS) + w, one wave per row.
// The slice of v goes to LDS by LDS-DMA first; the row segment of A (NCH
// chunks per lane per round) is issued after it, its addresses depending on an
// opaque zero, so the sum of squares waits only for the copy and runs while
// the row is in flight.  The column split doubles (or quadruples) the blocks
// of a small rank, so the read of A covers the whole chip.
// Block 0 also clears n_zero counters (the down projection's tile counters).
constexpr int K1_WAVES = 8;
constexpr int K1_THREADS = K1_WAVES * WAVE;

template <int PT, int NCH>
__global__ void __launch_bounds__(K1_THREADS)
k_predict_t(const void* __restrict__ A, int r, int d, int KS, const float* __restrict__ v, int glue,
            float* __restrict__ ss_out, float* __restrict__ t_part, int32_t* __restrict__ zero, int n_zero) {
  extern __shared__ float smem[];
  __shared__ float red[K1_WAVES];
  constexpr int EPL = Tr<PT>::EPL, TW = WAVE * EPL;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int ks = blockIdx.x % KS, grp = blockIdx.x / KS;
  const int row = grp * K1_WAVES + w;
  const size_t rowc = (size_t)min(row, r - 1);       // a wave without a row reads row r-1 and discards it
  const int ds = d / KS, off = ks * ds;               // this block's columns [off, off + ds)
  const int nch = (ds + TW - 1) / TW;
  float* xs = smem;                                   // v [dma_pad(ds)]

  if (blockIdx.x == 0)
    for (int k = tid; k < n_zero; k += K1_THREADS) zero[k] = 0;
  dma_f32(xs, v + off, ds, w, K1_WAVES, lane);
  const int z = opaque_zero();
  uint4 c[NCH];
#pragma unroll
  for (int q = 0; q < NCH; ++q)
    c[q] = ld_chunk<PT>(A, rowc + z, d, off + min(min(q, nch - 1) * TW + lane * EPL, ds - EPL));
  PI_ISSUE_FENCE();
  wait_vm_lds<NCH>();                                 // the copy, not the row
  __builtin_amdgcn_s_barrier();

  if (glue && grp == 0) {
    float ss = 0.f;
    for (int k = tid; k < ds / 4; k += K1_THREADS) {
      const float4 u = reinterpret_cast<const float4*>(xs)[k];
      ss = fmaf(u.x, u.x, ss);
      ss = fmaf(u.y, u.y, ss);
      ss = fmaf(u.z, u.z, ss);
      ss = fmaf(u.w, u.w, ss);
    }
    ss = wave_sum(ss);
    if (lane == 0) red[w] = ss;
    __syncthreads();
    if (tid == 0) {
      float tot = 0.f;
#pragma unroll
      for (int i = 0; i < K1_WAVES; ++i) tot += red[i];
      ss_out[ks] = tot;
    }
  }

  float a = 0.f;
#pragma unroll
  for (int q = 0; q < NCH; ++q) {
    const int e = q * TW + lane * EPL;
    const bool ok = q < nch && e < ds;
    const float p = chunk_dot<PT>(c[q], 1.f, xs + (ok ? e : 0));
    a += ok ? p : 0.f;
  }
  for (int q0 = NCH; q0 < nch; q0 += NCH) {            // slices longer than NCH chunks per lane
#pragma unroll
    for (int q = 0; q < NCH; ++q)
      c[q] = ld_chunk<PT>(A, rowc, d, off + min(min(q0 + q, nch - 1) * TW + lane * EPL, ds - EPL));
    PI_ISSUE_FENCE();
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      const int e = (q0 + q) * TW + lane * EPL;
      const bool ok = q0 + q < nch && e < ds;
      const float p = chunk_dot<PT>(c[q], 1.f, xs + (ok ? e : 0));
      a += ok ? p : 0.f;
    }
  }
  a = wave_sum(a);
  if (row < r && lane == 0) t_part[(size_t)ks * r + row] = a;
}

// ----------------------------------------------------------------------- K2
// Scores s_i = c_i + B[i] . t, threshold s_i > 0, and -- if FUSE -- the
// gathered up/gate GEMV with ReLU, ReGLU or Squared ReLU for the active
// neurons, in two phases.  t arrives as the predictor kernel's KS column-slice
// products; with a glue, t = inv (t_0 + ... + t_{KS-1}) and x' = v inv, inv =
// 1 / sqrt(ss / d + 1e-6) from the slices' sums of squares ss of v.
//  1. The rows of B.  The neurons are dealt to the blocks round-robin (so the
//     hot-first order spreads the frequently active rows evenly over the
//     blocks); wave w of block b owns neurons b + nb (w + K2_WAVES m).  The
//     block copies the slices of t into LDS by LDS-DMA ahead of the rows of B
//     and adds them up there (one barrier each side) while the first rows are
//     in flight.  Each wave loads RB = 16 / PCH rows (PCH 16-byte chunks per
//     lane each) before its first multiply, and appends the active ones to its
//     own list in LDS (ballot order: ascending within the wave).  No further
//     barrier: the waves stream B independently.
//  2. The block's active list (the waves' lists one after another), R rows
//     at a time, by all 256 lanes together: lane tid owns chunks tid + 256 j
//     (j < CPL) of every row, and holds its x' values for those chunks in
//     registers, loaded at the start.  Every load of a round is issued before
//     the first multiply; the lanes' partial dot products are summed per wave
//     and the waves' sums in a fixed order.  Wave 0 then applies the bias and
//     the activation and appends the neurons with h != 0 to the block's list
//     of (neuron, h) pairs: pair_id / pair_h [block][cap].  A neuron whose
//     ReLU output is 0 adds nothing to y, so the down projection reads only
//     the listed rows.
// cnt_blk[block] = active neurons of the block, cnt_blk[nb + block] = those
// with h != 0.  pmask (if given) gets the predictor's mask byte per neuron.
// Block b also writes its slice of x' to x_out / x_trace (if given).
// Hot-dense prefix: neurons i < hot are active without a prediction -- their
// rows of B are not read, their scores not written, their mask bytes are 1.
constexpr int K2_WAVES = 4;
constexpr int K2_THREADS = K2_WAVES * WAVE;

// Chunk slots of a lane loaded at once in a gather round (rows longer than
// 256 * 8 chunks take several groups), and rows per round: as many as keep
// NMAT * CG chunk loads per row at 16 per lane (at least 1).
template <int CPL> constexpr int k2_cg() { return CPL < 8 ? CPL : 8; }
template <int NMAT, int CPL> constexpr int k2_rows() {
  return (16 / (NMAT * k2_cg<CPL>())) < 1 ? 1 : 16 / (NMAT * k2_cg<CPL>());
}

// x' for the chunks a lane owns, in registers (EPL floats per chunk, and
// for Q4_0 the chunk's block sum).
template <int WT, int CPL>
struct XReg {
  float v[CPL][Tr<WT>::EPL];
  float bsum[CPL];
};

template <int WT, int CPL>
__device__ __forceinline__ void load_xreg(XReg<WT, CPL>& xr, const float* __restrict__ x, int nch, int tid) {
  constexpr int EPL = Tr<WT>::EPL;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = min(tid + K2_THREADS * j, nch - 1);
#pragma unroll
    for (int e = 0; e < EPL; e += 4) {
      const float4 v = *reinterpret_cast<const float4*>(x + (size_t)c * EPL + e);
      xr.v[j][e] = v.x;
      xr.v[j][e + 1] = v.y;
      xr.v[j][e + 2] = v.z;
      xr.v[j][e + 3] = v.w;
    }
  }
}

// x' = v inv in the registers, once the values have arrived.
template <int WT, int CPL>
__device__ __forceinline__ void xreg_scale(XReg<WT, CPL>& xr, float inv) {
  constexpr int EPL = Tr<WT>::EPL;
#pragma unroll
  for (int j = 0; j < CPL; ++j)
#pragma unroll
    for (int e = 0; e < EPL; ++e) xr.v[j][e] *= inv;
}

// The Q4_0 block sums of the chunks, once their values have arrived.
template <int WT, int CPL>
__device__ __forceinline__ void xreg_sums(XReg<WT, CPL>& xr) {
  if constexpr (WT == DT_Q4) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      float sum = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) sum += xr.v[j][e];
      xr.bsum[j] = sum;
    }
  }
}

// sum_j w_j * x_j over one chunk with x in registers (the chunk's EPL values).
// Q4_0: d (sum_j q_j x_j - 8 xsum), one conversion and one FMA per weight.
template <int DT>
__device__ __forceinline__ float chunk_dot_reg(uint4 c, float scale, const float* xv, float xsum) {
  if constexpr (DT == DT_F32) {
    float a = __uint_as_float(c.x) * xv[0];
    a = fmaf(__uint_as_float(c.y), xv[1], a);
    a = fmaf(__uint_as_float(c.z), xv[2], a);
    a = fmaf(__uint_as_float(c.w), xv[3], a);
    return a;
  } else if constexpr (DT == DT_F16) {
    const half8_t h = __builtin_bit_cast(half8_t, c);
    float a = (float)h[0] * xv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) a = fmaf((float)h[e], xv[e], a);
    return a;
  } else {
    const uint32_t wd[4] = {c.x, c.y, c.z, c.w};
    const uint32_t m = nib_mask();
    float a = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = wd[k] & m, hi = (wd[k] >> 4) & m;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        a = fmaf(ubyte_f(lo, b), xv[4 * k + b], a);
        a = fmaf(ubyte_f(hi, b), xv[4 * k + b + 16], a);
      }
    }
    return fmaf(-8.f, xsum, a) * scale;
  }
}

template <int PT, int WT, int ACT, bool FUSE, int PCH, int CPL>
__global__ void __launch_bounds__(K2_THREADS) __attribute__((amdgpu_waves_per_eu(2)))
k_score(const void* __restrict__ Bm, const float* __restrict__ pbias, const float* __restrict__ bias,
        const float* __restrict__ t_part, int KS, const float* __restrict__ ss_in, int f, int r,
        const void* __restrict__ gate_w, const uint16_t* __restrict__ gate_sc,
        const void* __restrict__ up_w, const uint16_t* __restrict__ up_sc,
        const float* __restrict__ vx, int d, float* __restrict__ x_out, float* __restrict__ x_trace,
        float* __restrict__ scores, uint8_t* __restrict__ pmask, int32_t* __restrict__ cnt_blk,
        int32_t* __restrict__ pair_id, float* __restrict__ pair_h, int cap, int hot) {
  constexpr int RB = 16 / PCH;                               // rows of B per batch
  constexpr int PEPL = Tr<PT>::EPL, PTW = WAVE * PEPL;
  constexpr int NMAT = act_nmat<ACT>();
  constexpr int R = k2_rows<NMAT, CPL>();                    // rows per gather round
  constexpr int EPL = Tr<WT>::EPL;
  extern __shared__ float smem[];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int nb = gridDim.x, b = blockIdx.x, NW = nb * K2_WAVES;
  const int g = b + nb * w;                                  // the wave's first neuron
  const int M = g < f ? (f - 1 - g) / NW + 1 : 0;            // neurons of this wave
  const int Mb = b < f ? (f - 1 - b) / NW + 1 : 0;           // wave 0 has the most: block-uniform trip count
  const int Mw = (f + NW - 1) / NW;                          // list capacity per wave (= Mb of block 0)
  const int mh = hot > g ? min(M, (hot - 1 - g) / NW + 1) : 0;   // the wave's neurons in the hot prefix
  const int dpr = dma_pad(r);
  float* ts = smem;                                          // the slices of t, then t [KS][dma_pad(r)]
  int* act = reinterpret_cast<int*>(smem + (size_t)KS * dpr);   // [K2_WAVES][Mw] active lists
  __shared__ int nact[K2_WAVES];
  __shared__ float red[2][K2_WAVES][R * NMAT];
  const int pch = (r + PTW - 1) / PTW;
  const int my_u = min(lane, RB - 1);                        // lane u < RB reports row u of the batch
  const int nch = (d + EPL - 1) / EPL;                       // chunks per gathered row

  // Rows past the wave's last neuron (all rows, for a wave without neurons)
  // and chunks past the row end load a clamped, valid address and are
  // discarded; no load sits in a branch.
  uint4 bc[RB][PCH];
  float pb = 0.f;
  auto nrow = [&](int m) __attribute__((always_inline)) { return min(g + NW * max(min(m, M - 1), 0), f - 1); };
  auto issue = [&](int m0, int q0, int z) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const size_t row = (size_t)(nrow(m0 + u) + z);
#pragma unroll
      for (int q = 0; q < PCH; ++q)
        bc[u][q] = ld_chunk<PT>(Bm, row, r, min(min(q0 + q, pch - 1) * PTW + lane * PEPL, r - PEPL));
    }
    if (q0 == 0) pb = pbias[nrow(m0 + my_u) + z];
    PI_ISSUE_FENCE();
  };

  // The slices of t go to LDS by LDS-DMA ahead of everything else; the first
  // rows of B next, their addresses depending on an opaque zero so they
  // cannot be hoisted; v for the gathers to registers last (it is needed
  // last).  The glue's scale inv = 1 / sqrt(mean(v^2) + 1e-6) comes from the
  // slices' sums of squares (inv = 1 without a glue).
  for (int k = 0; k < KS; ++k) dma_f32(ts + (size_t)k * dpr, t_part + (size_t)k * r, r, w, K2_WAVES, lane);
  float inv = 1.f;
  if (ss_in) {
    float tot = 0.f;
    for (int k = 0; k < KS; ++k) tot += ss_in[k];
    inv = 1.0f / sqrtf(tot / (float)d + 1e-6f);
  }
  // this block's slice of x' = v inv [kx0, kx1) for x_out / x_trace: its first
  // K2_THREADS elements are loaded with the copies and stored once they are in
  const int cx = (d + nb - 1) / nb, kx0 = min(d, b * cx), kx1 = min(d, kx0 + cx);
  const bool wx = x_out || x_trace;
  float vk = 0.f;
  if (wx && kx0 + tid < kx1) vk = vx[kx0 + tid];
  PI_ISSUE_FENCE();
  issue(mh, 0, opaque_zero());
  XReg<WT, CPL> xr;
  if constexpr (FUSE) load_xreg<WT, CPL>(xr, vx, nch, tid);
  PI_ISSUE_FENCE();
  // The copies of t (and v's slice) have arrived once no more than the loads
  // issued after them (the RB*PCH chunks of B, the bias, the x' chunks) are
  // outstanding; the barrier makes every wave's copies visible.
  wait_vm_lds<RB * PCH + 1 + (FUSE ? CPL * EPL / 4 : 0)>();
  __syncthreads();
  if (KS > 1 || ss_in) {
    // t = inv (t_0 + t_1 + ...), into the first slice
    for (int i = 4 * tid; i < r; i += 4 * K2_THREADS) {
      float4 a = *reinterpret_cast<const float4*>(ts + i);
      for (int k = 1; k < KS; ++k) {
        const float4 u = *reinterpret_cast<const float4*>(ts + (size_t)k * dpr + i);
        a.x += u.x;
        a.y += u.y;
        a.z += u.z;
        a.w += u.w;
      }
      a.x *= inv;
      a.y *= inv;
      a.z *= inv;
      a.w *= inv;
      *reinterpret_cast<float4*>(ts + i) = a;
    }
    __syncthreads();
  }
  if (wx && kx0 + tid < kx1) {
    const float xk = ss_in ? vk * inv : vk;                  // the same product as the gathers'
    if (x_out) x_out[kx0 + tid] = xk;
    if (x_trace) x_trace[kx0 + tid] = xk;
  }

  // the hot prefix: active without a score (no row of B is read, no score written)
  for (int m = lane; m < mh; m += WAVE) {
    act[w * Mw + m] = g + NW * m;
    if (pmask) pmask[g + NW * m] = 1;
  }
  int n_w = mh;                                              // this wave's active neurons so far
  for (int m0 = mh; m0 < Mb; m0 += RB) {
    float acc[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u) acc[u] = 0.f;
    for (int q0 = 0; q0 < pch; q0 += PCH) {
      if (q0 > 0) issue(m0, q0, 0);
#pragma unroll
      for (int u = 0; u < RB; ++u) {
#pragma unroll
        for (int q = 0; q < PCH; ++q) {
          const int e = (q0 + q) * PTW + lane * PEPL;
          const bool ok = q0 + q < pch && e < r;
          const float p = chunk_dot<PT>(bc[u][q], 1.f, ts + (ok ? e : 0));
          acc[u] += ok ? p : 0.f;
        }
      }
    }
    float dot = 0.f;
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const float su = wave_sum(acc[u]);
      if (lane == u) dot = su;
    }
    const int m = m0 + my_u;
    const bool rep = lane < RB && m < M;
    const int i = g + NW * m;
    const float sc = dot + pb;
    const bool on = rep && sc > 0.f;
    const uint64_t bal = __ballot(on);                       // lanes u < RB: rows in order
    if (on) act[w * Mw + n_w + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u))] = i;
    n_w += __popcll(bal);
    if (m0 + RB < Mb) issue(m0 + RB, 0, 0);                  // the next batch's rows of B
    if (rep) {
      if (scores) scores[i] = sc;
      if (pmask) pmask[i] = on ? 1 : 0;
    }
  }
  if (lane == 0) nact[w] = n_w;
  __syncthreads();
  int pre[K2_WAVES + 1];
  pre[0] = 0;
#pragma unroll
  for (int v = 0; v < K2_WAVES; ++v) pre[v + 1] = pre[v] + nact[v];
  const int n = pre[K2_WAVES];
  // entry a of the block's list: in the list of the wave whose prefix bounds it
  auto entry = [&](int a) __attribute__((always_inline)) {
    int ww = 0, base = 0;
#pragma unroll
    for (int v = 1; v < K2_WAVES; ++v)
      if (a >= pre[v]) { ww = v; base = pre[v]; }
    return act[ww * Mw + a - base];
  };

  int nz = 0;                                                // wave 0: neurons listed with h != 0
  if constexpr (FUSE) {
    if (ss_in) xreg_scale<WT, CPL>(xr, inv);                 // x' = v inv
    xreg_sums<WT, CPL>(xr);
    const void* w0 = (ACT == ACT_REGLU) ? gate_w : up_w;
    const uint16_t* s0 = (ACT == ACT_REGLU) ? gate_sc : up_sc;
    for (int a0 = 0, round = 0; a0 < n; a0 += R, ++round) {
      int rows[R];
#pragma unroll
      for (int u = 0; u < R; ++u) rows[u] = entry(min(a0 + u, n - 1));
      // wave 0, lane u < R: row u of the round and its bias (read with the rows)
      const int my_row = entry(min(a0 + min(lane, R - 1), n - 1));
      float bb = 0.f;
      constexpr int CG = k2_cg<CPL>();
      float part[R][NMAT];
#pragma unroll
      for (int u = 0; u < R; ++u)
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt) part[u][mt] = 0.f;
#pragma unroll
      for (int j0 = 0; j0 < CPL; j0 += CG) {
        uint4 c[R][NMAT][CG];
        float fs[R][NMAT][CG];
#pragma unroll
        for (int u = 0; u < R; ++u)
#pragma unroll
          for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
            for (int j = 0; j < CG; ++j) {
              const int cc = min(tid + K2_THREADS * (j0 + j), nch - 1);
              c[u][mt][j] = ld_chunk<WT>(mt ? up_w : w0, (size_t)rows[u], d, cc * EPL);
              fs[u][mt][j] = (WT == DT_Q4) ? ld_scale(mt ? up_sc : s0, (size_t)rows[u], d, cc * EPL) : 1.f;
            }
        if (j0 == 0 && w == 0) bb = bias[my_row];
        PI_ISSUE_FENCE();
#pragma unroll
        for (int u = 0; u < R; ++u)
#pragma unroll
          for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
            for (int j = 0; j < CG; ++j) {
              const float p = chunk_dot_reg<WT>(c[u][mt][j], fs[u][mt][j], xr.v[j0 + j], xr.bsum[j0 + j]);
              part[u][mt] += (tid + K2_THREADS * (j0 + j) < nch) ? p : 0.f;
            }
      }
      const int buf = round & 1;
#pragma unroll
      for (int u = 0; u < R; ++u)
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt) {
          const float v = wave_sum(part[u][mt]);
          if (lane == 0) red[buf][w][u * NMAT + mt] = v;
        }
      __syncthreads();
      if (w == 0) {
        // lane u < R: row u of the round (my_row)
        const int u = min(lane, R - 1);
        float z[NMAT];
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt) {
          float zz = 0.f;
#pragma unroll
          for (int v = 0; v < K2_WAVES; ++v) zz += red[buf][v][u * NMAT + mt];
          z[mt] = zz;
        }
        const float h = act_h<ACT>(z[0], bb, z[NMAT - 1]);
        const bool put = lane < R && a0 + lane < n && h != 0.f;
        const uint64_t hb = __ballot(put);
        if (put) {
          const int pos = nz + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(hb >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)hb, 0u));
          pair_id[(size_t)b * cap + pos] = my_row;
          pair_h[(size_t)b * cap + pos] = h;
        }
        nz += __popcll(hb);
      }
    }
  }
  if (tid == 0 && cnt_blk) {
    cnt_blk[b] = n;
    cnt_blk[nb + b] = nz;
  }
  if (wx)                                                    // the rest of the slice (few blocks)
    for (int k = kx0 + K2_THREADS + tid; k < kx1; k += K2_THREADS) {
      const float xk = ss_in ? vx[k] * inv : vx[k];
      if (x_out) x_out[k] = xk;
      if (x_trace) x_trace[k] = xk;
    }
}

// Up/gate over an explicit list (pi_sparse_ffn): h_list[j] for j < count, one
// list entry per wave at a time.  Entries outside [0, f) give h = 0 and read
// nothing.
template <int WT, int ACT, int WCH>
__global__ void __launch_bounds__(256)
k_up_list(const void* __restrict__ gate_w, const uint16_t* __restrict__ gate_sc,
          const void* __restrict__ up_w, const uint16_t* __restrict__ up_sc,
          const float* __restrict__ bias, const float* __restrict__ x, int d, int f,
          const int32_t* __restrict__ idx, const int32_t* __restrict__ count, float* __restrict__ h_list) {
  extern __shared__ float xs[];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE, W = blockDim.x / WAVE;
  const int cnt = min(max(*count, 0), f);
  if ((int)blockIdx.x * W >= cnt) return;
  if constexpr (WT == DT_Q4) {
    for (int k = tid; k < d; k += blockDim.x) xs[q4t_pos(k, d)] = x[k];
    for (int qb = tid; qb < d / 32; qb += blockDim.x) {
      float sum = 0.f;
      for (int j = 0; j < 32; ++j) sum += x[32 * qb + j];
      xs[d + qb] = sum;
    }
  } else {
    stage_f32<8>(xs, x, d, tid, blockDim.x);
  }
  __syncthreads();
  constexpr int NMAT = act_nmat<ACT>();
  const void* w0 = (ACT == ACT_REGLU) ? gate_w : up_w;
  const uint16_t* s0 = (ACT == ACT_REGLU) ? gate_sc : up_sc;
  for (int j = blockIdx.x * W + w; j < cnt; j += gridDim.x * W) {
    const int i = idx[j];
    float h = 0.f;
    if (i >= 0 && i < f) {
      const int rows[1] = {i};
      float z[1][NMAT];
      gather_rows<WT, WCH, NMAT, 1>(w0, s0, up_w, up_sc, rows, d, xs, lane, z);
      h = act_h<ACT>(z[0][0], bias[i], z[0][NMAT - 1]);
    }
    if (lane == 0) h_list[j] = h;
  }
}

// ----------------------------------------------------------------------- K3
// Down projection y = sum over listed neurons i of h_i * downT[i].
// Block (t, nc): column tile t (TWC 16-byte chunks = TWC*EPL columns) and
// neuron split nc of NC.  With the XCD-aware order, the blocks that the
// hardware places on one XCD (block ids congruent mod 8) own adjacent tiles,
// so the tiles that share a 128-byte line of a row share that XCD's L2.
// Each wave copies its share of the (neuron, h) entries into LDS -- in the
// stack, the per-block lists of the score kernel (wave s of S = 8*NC takes
// the lists of score blocks s, s + S, ...; a wave prefix sum of their counts
// places them; their first entries are read together with the counts, and
// only a list longer than that is read again after them); for pi_sparse_ffn, the caller's list with its h values
// (entries s, s + S, ... with h != 0) -- then gathers the tile's segments of
// those rows, RPW = 64 / TWC rows per wave-wide load and K3_LOADS loads per
// HBM round trip, accumulating in fp32 in list order.  The lanes of one chunk
// column are summed inside each 16-lane row, then the rows of all waves in a
// fixed order, and the tile's partial sums are written to y_part[nc][cols]
// with plain stores.
// With tile counters (zero at launch), the block that finishes a column tile
// last -- the blocks store their partial tiles with device-coherent stores,
// wait for them to be acknowledged and then count themselves with a
// device-scope atomic -- adds the NC partial tiles in split order,
// y = ((y_0 + y_1) + y_2) + ..., and writes y to y_out and x_res + y to v_out
// (those given).
constexpr int K3_WAVES = 8;
constexpr int K3_CAP = 1024;     // list entries per wave held at once
constexpr int K3_LOADS = 16;     // row segments per lane per HBM round trip (8 for Q4_0, whose
                                 // 32 values per segment need more registers to decode)
constexpr int K3_MAXLISTS = 64;  // score-block lists per wave (one per lane)

template <int WT, int TWC, bool EXPLICIT>
__global__ void __launch_bounds__(512)
k_down(const void* __restrict__ downT, const uint16_t* __restrict__ down_sc, int f, int d, int CT, int NC,
       int xcd_order, const int32_t* __restrict__ pair_id, const float* __restrict__ pair_h, int cap,
       const int32_t* __restrict__ idx, const int32_t* __restrict__ count, const float* __restrict__ h_list,
       const float* __restrict__ b_down, float* __restrict__ y_part, const int32_t* __restrict__ cnt_blk,
       int n_cnt_blk, int32_t* __restrict__ count_out, int32_t* __restrict__ count_out2,
       int32_t* __restrict__ nz_out, int32_t* __restrict__ tile_cnt, const float* __restrict__ x_res,
       float* __restrict__ y_out, float* __restrict__ v_out) {
  constexpr int EPL = Tr<WT>::EPL;
  constexpr int RPW = WAVE / TWC;                 // rows per wave-wide load
  constexpr int TCOL = TWC * EPL;                 // columns per tile
  // the waves' lists; after the gathers, the same memory holds the row sums
  // of every wave [K3_WAVES][4 rows][TCOL]
  static_assert(sizeof(float) * K3_WAVES * 4 * TCOL <= sizeof(int) * K3_WAVES * K3_CAP, "row sums fit the lists");
  __shared__ __attribute__((aligned(16))) int l_id[K3_WAVES][K3_CAP];
  __shared__ float l_h[K3_WAVES][K3_CAP];
  __shared__ int l_pre[K3_WAVES][K3_MAXLISTS];
  __shared__ int l_cnt[K3_WAVES][K3_MAXLISTS];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  const int nblk = CT * NC;
  int L = blockIdx.x;
  if (xcd_order) L = (blockIdx.x % 8) * (nblk / 8) + blockIdx.x / 8;
  const int tile = L % CT, nc = L / CT;
  const int S = NC * K3_WAVES, s = nc * K3_WAVES + w;
  const int q = lane % TWC, rl = lane / TWC;
  const int col = tile * TCOL + q * EPL;
  const int colc = min(col, d - EPL);             // lanes past d read a valid chunk, unused

  // block 0 also adds up the score kernel's per-block counts: active
  // neurons in cnt_blk[0, n), those with h != 0 in cnt_blk[n, 2n)
  __shared__ int cnt_red[2][K3_WAVES];
  const bool do_cnt = blockIdx.x == 0 && (count_out || count_out2 || nz_out);
  int cpart = 0, zpart = 0;
  if (do_cnt)
    for (int k = tid; k < n_cnt_blk; k += blockDim.x) {
      cpart += cnt_blk[k];
      zpart += cnt_blk[n_cnt_blk + k];
    }

  float acc[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) acc[j] = 0.f;
  float hsum = 0.f;                               // Q4_0: sum of h d over this lane's segments

  int n = 0;                                      // entries in this wave's list
  // gather the listed rows' segments: entry e = e0 + k*RPW + rl for wave-load
  // k; NL loads per round, all issued before the first multiply (entries past
  // the list repeat its last row with h = 0)
  auto batch = [&](auto nl_c, int e0) __attribute__((always_inline)) {
    constexpr int NL = decltype(nl_c)::value;
    uint4 c[NL];
    float sc[NL], hv[NL];
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int ec = min(e0 + k * RPW + rl, n - 1);
      const int row = l_id[w][ec];
      c[k] = ld_chunk<WT>(downT, (size_t)row, d, colc);
      sc[k] = (WT == DT_Q4) ? ld_scale(down_sc, (size_t)row, d, colc) : 1.f;
      hv[k] = l_h[w][ec];
    }
    PI_ISSUE_FENCE();
#pragma unroll
    for (int k = 0; k < NL; ++k) chunk_axpy<WT>(c[k], sc[k], (e0 + k * RPW + rl < n) ? hv[k] : 0.f, acc, hsum);
  };
  auto flush = [&]() __attribute__((always_inline)) {
    constexpr int NLMAX = WT == DT_Q4 ? 8 : K3_LOADS;
    for (int e0 = 0; e0 < n; e0 += NLMAX * RPW) {
      const int nl = (n - e0 + RPW - 1) / RPW;   // wave-uniform
      if (nl <= 4) batch(std::integral_constant<int, 4>{}, e0);
      else if (nl <= 8) batch(std::integral_constant<int, 8>{}, e0);
      else batch(std::integral_constant<int, NLMAX>{}, e0);
    }
    n = 0;
  };

  if constexpr (!EXPLICIT) {
    // the counts of this wave's score-block lists (block s + S i in lane i), and --
    // in the same round trip, before the counts are known -- the first `spec`
    // entries of every list (slot k of the 256 read ahead is entry k % spec of list
    // k / spec; spec is a power of two, at most the list capacity)
    const int nlw = n_cnt_blk > s ? (n_cnt_blk - 1 - s) / S + 1 : 0;     // <= K3_MAXLISTS
    int lg = 8;                                                          // log2(spec)
    while (lg > 0 && ((1 << lg) * nlw > 4 * WAVE || (1 << lg) > cap)) --lg;
    const int cl = lane < nlw ? cnt_blk[n_cnt_blk + s + S * lane] : 0;
    int sid[4];
    float sh[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int slot = k * WAVE + lane, li = slot >> lg, e = slot & ((1 << lg) - 1);
      const size_t at = li < nlw ? (size_t)(s + S * li) * cap + e : 0;   // a valid entry either way
      sid[k] = pair_id[at];
      sh[k] = pair_h[at];
    }
    PI_ISSUE_FENCE();
    const int incl = wave_scan(cl);
    l_pre[w][lane] = incl - cl;
    l_cnt[w][lane] = cl;
    const int ntot = lane_i(incl, WAVE - 1);
    // every entry read ahead (no list longer than spec) and the wave's list fits: place
    // them; otherwise the general path below reads every entry again
    const bool all_ahead = __ballot(cl > (1 << lg)) == 0 && ntot <= K3_CAP;
    if (all_ahead) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int slot = k * WAVE + lane, li = slot >> lg, e = slot & ((1 << lg) - 1);
        const int lic = min(li, K3_MAXLISTS - 1);
        if (li < nlw && e < l_cnt[w][lic]) {
          l_id[w][l_pre[w][lic] + e] = sid[k];
          l_h[w][l_pre[w][lic] + e] = sh[k];
        }
      }
      n = ntot;
      flush();
    } else {
      // entries e0 .. e0 + K3_CAP at a time; entry e is in the list i whose
      // prefix bounds it (a search over the nlw prefixes), at offset e - pre[i]
      for (int e0 = 0; e0 < ntot; e0 += K3_CAP) {
        const int ne = min(K3_CAP, ntot - e0);
        for (int k0 = 0; k0 < ne; k0 += 4 * WAVE) {
          size_t slot[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int e = e0 + min(k0 + k * WAVE + lane, ne - 1);
            int lo = 0;
#pragma unroll
            for (int step = K3_MAXLISTS / 2; step >= 1; step >>= 1)
              if (lo + step < nlw && l_pre[w][min(lo + step, K3_MAXLISTS - 1)] <= e) lo += step;
            slot[k] = (size_t)(s + S * lo) * cap + (e - l_pre[w][lo]);
          }
          int id4[4];
          float h4[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            id4[k] = pair_id[slot[k]];
            h4[k] = pair_h[slot[k]];
          }
          PI_ISSUE_FENCE();
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int e = k0 + k * WAVE + lane;
            if (e < ne) {
              l_id[w][e] = id4[k];
              l_h[w][e] = h4[k];
            }
          }
        }
        n = ne;
        flush();
      }
    }
  } else {
    const int cnt = min(max(*count, 0), f);
    for (int p0 = s; p0 < cnt; p0 += S * WAVE) {
      const int p = min(p0 + S * lane, cnt - 1);
      const int id = idx[p];
      const float hl = h_list[p];
      const bool on = p0 + S * lane < cnt && id >= 0 && id < f && hl != 0.f;   // h = 0 adds nothing
      const uint64_t bal = __ballot(on);
      if (bal == 0) continue;
      if (n > K3_CAP - WAVE) flush();
      if (on) {
        const int pos = n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        l_id[w][pos] = id;
        l_h[w][pos] = hl;
      }
      n += __popcll(bal);
    }
    if (n > 0) flush();
  }
  if constexpr (WT == DT_Q4) {
#pragma unroll
    for (int j = 0; j < EPL; ++j) acc[j] = fmaf(-8.f, hsum, acc[j]);
  }

  // Sum the row lanes of each chunk column (lanes with equal lane % TWC hold
  // the same columns) inside each 16-lane row; the last TWC lanes of each row
  // then write their sums, and the block adds the 4 rows of its 8 waves.
#pragma unroll
  for (int j = 0; j < EPL; ++j) acc[j] = row_group_sum<TWC>(acc[j]);
  __syncthreads();                                // every wave is done with its list
  float* rsum = reinterpret_cast<float*>(&l_id[0][0]);   // [K3_WAVES][4][TCOL]
  if ((lane & 15) >= 16 - TWC) {
    float* dst = rsum + ((size_t)w * 4 + lane / 16) * TCOL + (lane % TWC) * EPL;
#pragma unroll
    for (int j = 0; j < EPL; j += 4) *reinterpret_cast<float4*>(dst + j) = make_float4(acc[j], acc[j + 1], acc[j + 2], acc[j + 3]);
  }
  if (do_cnt) {
    cpart = wave_sum(cpart);
    zpart = wave_sum(zpart);
    if (lane == 0) {
      cnt_red[0][w] = cpart;
      cnt_red[1][w] = zpart;
    }
  }
  __syncthreads();
  if (do_cnt && tid == 0) {
    int tot = 0, tz = 0;
    for (int i = 0; i < K3_WAVES; ++i) {
      tot += cnt_red[0][i];
      tz += cnt_red[1][i];
    }
    if (count_out) *count_out = tot;
    if (count_out2) *count_out2 = tot;
    if (nz_out) *nz_out = tz;
  }
  for (int cc = tid; cc < TCOL; cc += blockDim.x) {
    const int cg = tile * TCOL + cc;
    if (cg >= d) continue;
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < K3_WAVES * 4; ++i) v += rsum[(size_t)i * TCOL + cc];
    if (b_down && nc == 0) v += b_down[cg];
    if (tile_cnt)   // device-coherent store: read by the tile's last block, maybe on another XCD
      __hip_atomic_store(&y_part[(size_t)nc * d + cg], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      y_part[(size_t)nc * d + cg] = v;
  }
  if (tile_cnt) {
    // Every store of the partial tile is acknowledged (vmcnt 0) before the
    // block is counted; the last block reads the partials with device-coherent
    // loads.  This keeps the whole-L2 write-back and invalidation of an
    // agent-scope release/acquire fence pair off the path.
    __shared__ int last;
    wait_vm_lds<0>();
    __syncthreads();
    if (tid == 0) last = __hip_atomic_fetch_add(&tile_cnt[tile], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == NC - 1;
    __syncthreads();
    if (last) {
      for (int cc = tid; cc < TCOL; cc += blockDim.x) {
        const int cg = tile * TCOL + cc;
        if (cg >= d) continue;
        float y = __hip_atomic_load(&y_part[cg], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int p = 1; p < NC; ++p)
          y += __hip_atomic_load(&y_part[(size_t)p * d + cg], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (y_out) y_out[cg] = y;
        if (v_out) v_out[cg] = x_res[cg] + y;
      }
    }
  }
}


// --------------------------------------------------------------- small ones
// Ascending list of the neurons whose mask byte is set (single block of 1024
// threads): idx[0..count), *count (and *count2, *count3 if not NULL).  The mask holds
// 0 or 1 per neuron and is read 16 bytes at a time, the ragged tail bytewise.  Each thread takes 16
// bytes per round; a DPP scan of the per-thread counts inside each wave and a
// scan of the wave totals give each thread its output position.
__global__ void __launch_bounds__(1024)
k_compact(const uint8_t* __restrict__ mask, int f, int32_t* __restrict__ idx, int32_t* __restrict__ count,
          int32_t* __restrict__ count2, int32_t* __restrict__ count3) {
  __shared__ int wsum[16];
  __shared__ int base_s;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE, W = blockDim.x / WAVE;
  const int ngrp = (f + 15) / 16;
  if (tid == 0) base_s = 0;
  __syncthreads();
  for (int g0 = 0; g0 < ngrp; g0 += blockDim.x) {
    const int grp = g0 + tid;
    uint32_t bits = 0;
    if (grp * 16 + 16 <= f) {
      const uint4 v = reinterpret_cast<const uint4*>(mask)[grp];
      auto b4 = [](uint32_t x) __attribute__((always_inline)) { return ((x & 0x01010101u) * 0x01020408u) >> 24; };
      bits = b4(v.x) | (b4(v.y) << 4) | (b4(v.z) << 8) | (b4(v.w) << 12);
    } else if (grp < ngrp) {
      for (int j = 0; j < f - grp * 16; ++j) bits |= (mask[grp * 16 + j] ? 1u : 0u) << j;   // ragged tail, bytewise
    }
    const int c = __popc(bits);
    const int inc = wave_scan(c);
    if (lane == WAVE - 1) wsum[w] = inc;
    __syncthreads();
    int wbase = 0;
    for (int k = 0; k < w; ++k) wbase += wsum[k];
    int pos = base_s + wbase + inc - c;
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      idx[pos++] = grp * 16 + b;
    }
    __syncthreads();
    if (tid == 0) {
      int tot = 0;
      for (int k = 0; k < W; ++k) tot += wsum[k];
      base_s += tot;
    }
    __syncthreads();
  }
  if (tid == 0) {
    *count = base_s;
    if (count2) *count2 = base_s;
    if (count3) *count3 = base_s;
  }
}

// *out = *out2 = sum of n per-block counts (single block of 256 threads; either may be NULL)
__global__ void __launch_bounds__(256)
k_sum_counts(const int32_t* __restrict__ cnt, int n, int32_t* __restrict__ out, int32_t* __restrict__ out2) {
  __shared__ int red[4];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  int c = 0;
  for (int k = tid; k < n; k += blockDim.x) c += cnt[k];
  c = wave_sum(c);
  if (lane == 0) red[w] = c;
  __syncthreads();
  if (tid == 0) {
    const int tot = red[0] + red[1] + red[2] + red[3];
    if (out) *out = tot;
    if (out2) *out2 = tot;
  }
}

// y = sum of np partial vectors of n floats, added in order
__global__ void k_finalize(const float* __restrict__ y_part, int np, float* __restrict__ y, int n) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k < n) {
    float v = y_part[k];
    for (int p = 1; p < np; ++p) v += y_part[(size_t)p * n + k];
    y[k] = v;
  }
}

// out = glue(x, y) with y given as np partials: single block, same operation
// order as K1's glue.
__global__ void __launch_bounds__(256)
k_glue_out(const float* __restrict__ x, const float* __restrict__ y_part, int np, float* __restrict__ out, int d) {
  extern __shared__ float vs[];
  __shared__ float red[16];
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE, W = blockDim.x / WAVE;
  float ss = stage_residual(vs, x, y_part, np, d, tid, blockDim.x);
  ss = wave_sum(ss);
  if (lane == 0) red[w] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int i = 0; i < W; ++i) tot += red[i];
  const float inv = 1.0f / sqrtf(tot / (float)d + 1e-6f);
  for (int k = tid; k < d; k += blockDim.x) out[k] = vs[k] * inv;
}

}  // namespace pik
