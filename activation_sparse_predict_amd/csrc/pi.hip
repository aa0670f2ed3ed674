// Host side of the C ABI declared in include/pi.h: argument validation,
// workspace layout, launch configuration and kernel dispatch.
#include "pi.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "pi_batch.hpp"
#include "pi_kernels.hpp"

namespace {

using namespace pik;

constexpr size_t kAlign = 256;

size_t align_up(size_t v, size_t a = kAlign) { return (v + a - 1) / a * a; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ------------------------------------------------------------------ checks
pi_status check_mat(const pi_mat& m, int32_t dtype) {
  if (!m.w || !aligned(m.w, 16)) return PI_EINVAL;
  if (dtype == PI_Q4_0) {
    if (!m.scale || !aligned(m.scale, 4)) return PI_EINVAL;
  }
  return PI_OK;
}

constexpr int kMaxD = 16384;
constexpr int kMaxRank = 4096;
constexpr int kMaxFfn = 1 << 21;   // the score kernel keeps each wave's active list in LDS

pi_status check_layer(const pi_layer* L) {
  if (!L) return PI_EINVAL;
  if (L->d <= 0 || L->ffn <= 0 || L->rank <= 0) return PI_EINVAL;
  if (L->d % 64 != 0 || L->rank % 64 != 0) return PI_EINVAL;
  if (L->act != PI_RELU && L->act != PI_REGLU && L->act != PI_RELU2) return PI_EINVAL;
  if (L->w_dtype != PI_F32 && L->w_dtype != PI_F16 && L->w_dtype != PI_Q4_0) return PI_EINVAL;
  if (L->p_dtype == PI_Q4_0) return PI_EUNSUPPORTED;
  if (L->d > kMaxD || L->rank > kMaxRank) return PI_EUNSUPPORTED;   // vectors staged whole in LDS
  if (L->ffn > kMaxFfn) return PI_EUNSUPPORTED;
  if (L->p_dtype != PI_F32 && L->p_dtype != PI_F16) return PI_EINVAL;
  if (!L->A || !L->B || !L->bias) return PI_EINVAL;
  if (!aligned(L->A, 16) || !aligned(L->B, 16) || !aligned(L->bias, 16)) return PI_EINVAL;
  pi_status s;
  if ((s = check_mat(L->up, L->w_dtype)) != PI_OK) return s;
  if ((s = check_mat(L->downT, L->w_dtype)) != PI_OK) return s;
  if (L->act == PI_REGLU && (s = check_mat(L->gate, L->w_dtype)) != PI_OK) return s;
  if (L->b_down && !aligned(L->b_down, 4)) return PI_EINVAL;
  if (L->pbias && !aligned(L->pbias, 16)) return PI_EINVAL;
  if (L->hot < 0 || L->hot > L->ffn) return PI_EINVAL;
  return PI_OK;
}

pi_status check_batch(int32_t batch) {
  if (batch < 1 || batch > 32) return PI_EINVAL;
  return PI_OK;
}

// the batched path keeps a split of the union list in LDS
pi_status check_batched_ffn(const pi_layer* L, int32_t batch) {
  return (batch > 1 && L->ffn > pib::BD_MAXF) ? PI_EUNSUPPORTED : PI_OK;
}

// -------------------------------------------------------------- workspace
struct Dims {
  int d = 0, fmax = 0, rmax = 0;
  int zmat = 0;      // z vectors of the Q4_0 K-split up GEMM: 0 without Q4_0 layers, else 1 (2 with ReGLU)
};

constexpr int kMaxParts = 8;       // neuron splits of the down projection (partial y vectors)
constexpr int kK1MaxSplit = 4;     // column slices of the predictor's first product
constexpr int kMaxTiles = 1024;    // column tiles of the down projection (at most 512 for d <= 16384)
constexpr int kK2Grid = 512;   // two per compute unit of an MI355X

int epl_of(int dt) { return dt == PI_F32 ? 4 : (dt == PI_F16 ? 8 : 32); }
int cdiv(int a, int b) { return (a + b - 1) / b; }

// Grid size of the score kernel (one active count per block), at most kK2Grid,
// the capacity of each block's (neuron, h) list, and the entries of all lists.
int k2_blocks_for(int ffn) { return std::max(1, std::min(kK2Grid, cdiv(ffn, 2 * K2_WAVES))); }   // >= 2 rows per wave
int k2_blocks_max(int ffn) { return k2_blocks_for(ffn); }
int k2_cap(int ffn) { return K2_WAVES * cdiv(ffn, k2_blocks_for(ffn) * K2_WAVES); }
size_t k2_pairs_max(int ffn) { return (size_t)k2_blocks_for(ffn) * k2_cap(ffn); }
// blocks of the batched score kernel: one tile of 32 neurons each
int bscore_blocks(int ffn) { return cdiv(ffn, pib::BM); }   // 32-neuron tiles of the batched score kernel

struct WsLayout {
  size_t t, v, ss, tcnt, xbuf, ybuf, mask, pmask, h, pid, ph, cnt, misc;
  // batched path (batch > 1)
  size_t xh, xl, tpart, th, tl, mnm, ulist, h32, rsc, zpart;
  size_t total;
  size_t xs, ys;   // sizes of one x / one y buffer
};

constexpr int kBatchM = pib::BM;      // padded batch rows of the batched GEMMs
// blocks of the batched up GEMMs, which loop over the union's tiles (a multiple of
// every K-split count, so a block of the K-split GEMM keeps its split)
constexpr int kUpGrid = 512;
static_assert(kUpGrid % pib::BU_KSMAX == 0, "blocks keep their K split");
constexpr int kMaxKSplit = 16;        // K splits of the batched predictor's first GEMM
static_assert(kMaxKSplit <= pib::BT_KS, "k_bsplit_t holds every split of a value");

WsLayout layout(const Dims& D, int batch) {
  WsLayout w{};
  size_t o = 0;
  const size_t fpad = (size_t)cdiv(D.fmax, 16) * 16;
  w.xs = align_up(sizeof(float) * (size_t)D.d * batch);
  w.ys = align_up(sizeof(float) * (size_t)D.d * (batch > 1 ? pib::bd_splits(D.d) * kBatchM : kMaxParts));
  w.t = o;    o += align_up(sizeof(float) * (size_t)D.rmax * std::max(batch, kK1MaxSplit));
  w.v = o;    o += align_up(sizeof(float) * (size_t)D.d);              // x' + y of a layer (batch 1)
  w.ss = o;   o += align_up(sizeof(float) * kK1MaxSplit);              // its slices' sums of squares
  w.tcnt = o; o += align_up(sizeof(int32_t) * kMaxTiles);             // the down projection's tile counters
  w.xbuf = o; o += w.xs * 2;
  w.ybuf = o; o += w.ys * 2;
  w.mask = o; o += align_up(fpad);                       // one byte per neuron (the union when batch > 1)
  w.pmask = o; o += align_up(fpad);                      // the predictor's mask for a trace list (batch 1)
  w.h = o;    o += align_up(sizeof(float) * (size_t)D.fmax);
  // the score kernel's per-block (neuron, h) lists [blocks][cap] (batch 1)
  w.pid = o;  o += align_up(sizeof(int32_t) * k2_pairs_max(D.fmax));
  w.ph = o;   o += align_up(sizeof(float) * k2_pairs_max(D.fmax));
  // per-block counts: active neurons, then those with h != 0 (batch 1)
  w.cnt = o;  o += align_up(sizeof(int32_t) * (size_t)std::max(2 * k2_blocks_max(D.fmax), bscore_blocks(D.fmax)));
  w.misc = o; o += kAlign;
  if (batch > 1) {
    w.xh = o;    o += align_up(sizeof(uint16_t) * (size_t)kBatchM * D.d);
    w.xl = o;    o += align_up(sizeof(uint16_t) * (size_t)kBatchM * D.d);
    w.tpart = o; o += align_up(sizeof(float) * (size_t)kMaxKSplit * kBatchM * D.rmax);
    w.th = o;    o += align_up(sizeof(uint16_t) * (size_t)kBatchM * D.rmax);
    w.tl = o;    o += align_up(sizeof(uint16_t) * (size_t)kBatchM * D.rmax);
    w.mnm = o;   o += align_up((size_t)kBatchM * D.fmax);
    w.ulist = o; o += align_up(sizeof(int32_t) * (size_t)D.fmax);
    w.h32 = o;   o += align_up(sizeof(float) * (size_t)kBatchM * pib::h_stride(D.fmax));
    w.rsc = o;   o += align_up(sizeof(float) * 3 * kBatchM);   // row scales of x and t, row maxima of h
    // the K splits of the Q4_0 up GEMM's z [KS][nmat][ffn padded to 32][32]
    w.zpart = o; o += align_up(sizeof(float) * (size_t)pib::bu_ks(D.d) * D.zmat * cdiv(D.fmax, kBatchM) * kBatchM * kBatchM);
  }
  w.total = o;
  return w;
}

struct Ws {
  float* t;
  float* v;
  float* ss;
  int32_t* tcnt;
  float* x[2];
  float* y[2];
  uint8_t* mask;
  uint8_t* pmask;
  float* h;
  int32_t* pid;
  float* ph;
  int32_t* cnt;
  int32_t* misc;
  _Float16 *xh, *xl, *th, *tl;
  float *h32, *sx, *st, *zpart;
  uint32_t* hmax;
  float* tpart;
  uint8_t* mnm;
  int32_t* ulist;
};

Ws carve(void* base, const WsLayout& L) {
  char* b = static_cast<char*>(base);
  Ws w{};
  w.t = reinterpret_cast<float*>(b + L.t);
  w.v = reinterpret_cast<float*>(b + L.v);
  w.ss = reinterpret_cast<float*>(b + L.ss);
  w.tcnt = reinterpret_cast<int32_t*>(b + L.tcnt);
  w.x[0] = reinterpret_cast<float*>(b + L.xbuf);
  w.x[1] = reinterpret_cast<float*>(b + L.xbuf + L.xs);
  w.y[0] = reinterpret_cast<float*>(b + L.ybuf);
  w.y[1] = reinterpret_cast<float*>(b + L.ybuf + L.ys);
  w.mask = reinterpret_cast<uint8_t*>(b + L.mask);
  w.pmask = reinterpret_cast<uint8_t*>(b + L.pmask);
  w.h = reinterpret_cast<float*>(b + L.h);
  w.pid = reinterpret_cast<int32_t*>(b + L.pid);
  w.ph = reinterpret_cast<float*>(b + L.ph);
  w.cnt = reinterpret_cast<int32_t*>(b + L.cnt);
  w.misc = reinterpret_cast<int32_t*>(b + L.misc);
  if (L.xh) {
    w.xh = reinterpret_cast<_Float16*>(b + L.xh);
    w.xl = reinterpret_cast<_Float16*>(b + L.xl);
    w.tpart = reinterpret_cast<float*>(b + L.tpart);
    w.th = reinterpret_cast<_Float16*>(b + L.th);
    w.tl = reinterpret_cast<_Float16*>(b + L.tl);
    w.mnm = reinterpret_cast<uint8_t*>(b + L.mnm);
    w.ulist = reinterpret_cast<int32_t*>(b + L.ulist);
    w.h32 = reinterpret_cast<float*>(b + L.h32);
    w.sx = reinterpret_cast<float*>(b + L.rsc);
    w.st = w.sx + kBatchM;
    w.hmax = reinterpret_cast<uint32_t*>(w.st + kBatchM);
    w.zpart = reinterpret_cast<float*>(b + L.zpart);
  }
  return w;
}

bool dims_of(const pi_layer* layers, int32_t n, Dims* D) {
  if (!layers || n <= 0) return false;
  for (int i = 0; i < n; ++i) {
    if (check_layer(&layers[i]) != PI_OK) return false;
    if (i > 0 && layers[i].d != layers[0].d) return false;
    D->d = layers[0].d;
    D->fmax = std::max(D->fmax, layers[i].ffn);
    D->rmax = std::max(D->rmax, layers[i].rank);
    if (layers[i].w_dtype == PI_Q4_0) D->zmat = std::max(D->zmat, layers[i].act == PI_REGLU ? 2 : 1);
  }
  return true;
}

// ---------------------------------------------------------- launch shapes
constexpr int kThreads = 256;

// 16-byte chunks per lane that one wave-wide pass over a row of n elements takes
int chunks_of(int n, int dt) { return cdiv(n, WAVE * epl_of(dt)); }

// Smallest supported per-round chunk count >= n (the largest if none is; the
// kernel then loops over rounds).  Loads of a round are issued unconditionally,
// so an exact fit avoids reading chunks twice.
template <size_t K>
int pick(const int (&opts)[K], int n) {
  for (size_t i = 0; i < K; ++i)
    if (opts[i] >= n) return opts[i];
  return opts[K - 1];
}

// K1: one wave per row of A and column slice; the slices multiply the blocks
// of a small rank up to about 256 (at most 4 slices, and no more than the
// score kernel's LDS copies of t allow).
constexpr int kK1Nch[] = {2, 4, 8, 12, 16, 24};
int k1_split(int r) {
  int ks = 1;
  while (ks < kK1MaxSplit && cdiv(r, K1_WAVES) * ks * 2 <= 256 && ks * 2 * dma_pad(r) <= 16384) ks *= 2;
  return ks;
}
int k1_blocks(int r) { return std::max(1, cdiv(r, K1_WAVES)) * k1_split(r); }

// K2: chunks per lane per row of B held at once (1 or 2)
int k2_pch_of(int rank, int p_dtype) { return chunks_of(rank, p_dtype) <= 1 ? 1 : 2; }
int k2_pch(const pi_layer* L) { return k2_pch_of(L->rank, L->p_dtype); }
// Chunks per lane of a gathered row (each of the block's 256 lanes owns
// chunks tid + 256 j): the smallest supported power of two that covers the row.
constexpr int kCplF32[] = {1, 2, 4, 8, 16};
constexpr int kCplF16[] = {1, 2, 4, 8};
constexpr int kCplQ4[] = {1, 2};
int k2_cpl(const pi_layer* L) {
  const int n = cdiv(L->d / epl_of(L->w_dtype), K2_THREADS);
  return L->w_dtype == PI_F32 ? pick(kCplF32, n) : L->w_dtype == PI_F16 ? pick(kCplF16, n) : pick(kCplQ4, n);
}
int k2_blocks(const pi_layer* L) { return k2_blocks_for(L->ffn); }

// K3: tiles of TWC = 4 chunks per row (64-byte row segments: one request per
// row and tile, half an L2 line, the other half read by the neighbouring tile
// on the same XCD), 8 chunks (a whole 128-byte line) for rows of 768 chunks
// or more, and for Q4_0 rows of 384 chunks or more (measured on MI355X: 15%
// faster at d = 8192 fp16, 23% at d = 7168, 24% at d = 12288 Q4_0, 12% slower
// at d = 4096 fp16), fewer when the row is short, and NC neuron splits so that
// the grid has at most 256 blocks of 8 waves (one round on the CUs).  Wider
// tiles scan the mask fewer times per row but give fewer blocks; narrower ones
// multiply the DRAM requests per byte.
struct K3Shape {
  int twc, ct, nc;
};
K3Shape k3_shape(int d, int dt) {
  const int nchunks = d / epl_of(dt);
  K3Shape s;
  const bool wide = nchunks >= 768 || (dt == PI_Q4_0 && nchunks >= 384);
  s.twc = wide ? 8 : nchunks >= 64 ? 4 : nchunks >= 32 ? 2 : 1;
  s.ct = cdiv(nchunks, s.twc);
  s.nc = std::max(1, std::min(kMaxParts, 256 / s.ct));
  return s;
}

// ---------------------------------------------------------------- dispatch
struct K1Args {
  const float* v;        // the layer's input before the glue [d]
  bool glue;             // normalise it (the sums of squares go to ss)
  float* ss;             // [k1_split]
  float* t_part;         // [k1_split][rank]
  int32_t* zero;         // counters to clear, or NULL
  int n_zero;
};

template <int PT, int NCH>
void launch_k1_t(const pi_layer* L, const K1Args& a, hipStream_t st) {
  const int ks = k1_split(L->rank), ds = L->d / ks;
  hipLaunchKernelGGL((k_predict_t<PT, NCH>), dim3(k1_blocks(L->rank)), dim3(K1_WAVES * WAVE),
                     sizeof(float) * (size_t)dma_pad(ds), st, L->A, L->rank, L->d, ks, a.v, a.glue ? 1 : 0, a.ss,
                     a.t_part, a.zero, a.zero ? a.n_zero : 0);
}

template <int PT>
void launch_k1_p(const pi_layer* L, const K1Args& a, hipStream_t st) {
  switch (pick(kK1Nch, chunks_of(L->d / k1_split(L->rank), L->p_dtype))) {
    case 2: return launch_k1_t<PT, 2>(L, a, st);
    case 4: return launch_k1_t<PT, 4>(L, a, st);
    case 8: return launch_k1_t<PT, 8>(L, a, st);
    case 12: return launch_k1_t<PT, 12>(L, a, st);
    case 16: return launch_k1_t<PT, 16>(L, a, st);
    default: return launch_k1_t<PT, 24>(L, a, st);
  }
}

void k1(const pi_layer* L, const K1Args& a, hipStream_t st) {
  if (L->p_dtype == PI_F32)
    launch_k1_p<DT_F32>(L, a, st);
  else
    launch_k1_p<DT_F16>(L, a, st);
}

struct K2Args {
  const float* t_part; // the predictor kernel's slices of t [k1_split][rank]
  const float* ss;     // their sums of squares of v, or NULL (no glue: x' = v)
  const float* v;      // v (the fused gathers take x' = v inv)
  float* x_out;        // x', or NULL
  float* x_trace;
  float* scores;
  uint8_t* pmask;      // the predictor's mask byte per neuron, or NULL
  int32_t* cnt;        // [2 * blocks]: active neurons, then those with h != 0
  int32_t* pid;        // [blocks][cap] (neuron, h) lists of the fused gathers
  float* ph;
};

template <int PT, int WT, int ACT, bool FUSE, int PCH, int CPL>
void launch_k2_t(const pi_layer* L, const K2Args& a, hipStream_t st) {
  const int nb = k2_blocks(L);
  const int ks = k1_split(L->rank);
  const size_t lds = sizeof(float) * ((size_t)ks * dma_pad(L->rank) + (size_t)K2_WAVES * cdiv(L->ffn, nb * K2_WAVES));
  hipLaunchKernelGGL((k_score<PT, WT, ACT, FUSE, PCH, CPL>), dim3(nb), dim3(K2_THREADS), lds, st,
                     L->B, L->pbias ? L->pbias : L->bias, L->bias, a.t_part, ks, a.ss, L->ffn, L->rank, L->gate.w,
                     L->gate.scale, L->up.w, L->up.scale, a.v, L->d, a.x_out, a.x_trace, a.scores, a.pmask, a.cnt,
                     a.pid, a.ph, k2_cap(L->ffn), L->hot);
}

template <int PT, int WT, int ACT, int PCH>
void launch_k2_fused(const pi_layer* L, const K2Args& a, hipStream_t st) {
  const int cpl = k2_cpl(L);
  if constexpr (WT == DT_Q4) {
    if (cpl == 1) return launch_k2_t<PT, WT, ACT, true, PCH, 1>(L, a, st);
    return launch_k2_t<PT, WT, ACT, true, PCH, 2>(L, a, st);
  } else {
    if (cpl == 1) return launch_k2_t<PT, WT, ACT, true, PCH, 1>(L, a, st);
    if (cpl == 2) return launch_k2_t<PT, WT, ACT, true, PCH, 2>(L, a, st);
    if (cpl == 4) return launch_k2_t<PT, WT, ACT, true, PCH, 4>(L, a, st);
    if constexpr (WT == DT_F16) {
      return launch_k2_t<PT, WT, ACT, true, PCH, 8>(L, a, st);
    } else {
      if (cpl == 8) return launch_k2_t<PT, WT, ACT, true, PCH, 8>(L, a, st);
      return launch_k2_t<PT, WT, ACT, true, PCH, 16>(L, a, st);
    }
  }
}

template <int PT, int WT, int PCH>
void launch_k2_act(const pi_layer* L, const K2Args& a, hipStream_t st) {
  switch (L->act) {
    case PI_REGLU: return launch_k2_fused<PT, WT, ACT_REGLU, PCH>(L, a, st);
    case PI_RELU2: return launch_k2_fused<PT, WT, ACT_RELU2, PCH>(L, a, st);
    default: return launch_k2_fused<PT, WT, ACT_RELU, PCH>(L, a, st);
  }
}

template <int PT, int PCH>
void launch_k2_p(const pi_layer* L, bool fuse, const K2Args& a, hipStream_t st) {
  if (!fuse) return launch_k2_t<PT, DT_F32, ACT_RELU, false, PCH, 1>(L, a, st);
  switch (L->w_dtype) {
    case PI_F32: return launch_k2_act<PT, DT_F32, PCH>(L, a, st);
    case PI_F16: return launch_k2_act<PT, DT_F16, PCH>(L, a, st);
    default: return launch_k2_act<PT, DT_Q4, PCH>(L, a, st);
  }
}

void k2(const pi_layer* L, bool fuse_up, const K2Args& a, hipStream_t st) {
  const bool p2 = k2_pch(L) == 2;
  if (L->p_dtype == PI_F32)
    p2 ? launch_k2_p<DT_F32, 2>(L, fuse_up, a, st) : launch_k2_p<DT_F32, 1>(L, fuse_up, a, st);
  else
    p2 ? launch_k2_p<DT_F16, 2>(L, fuse_up, a, st) : launch_k2_p<DT_F16, 1>(L, fuse_up, a, st);
}

struct K3Args {
  const int32_t* pid;        // list mode: the score kernel's per-block (neuron, h) lists
  const float* ph;
  int cap;
  const int32_t* idx;        // explicit mode
  const int32_t* count;
  const float* h_list;
  float* y_part;             // [nc][d]
  const int32_t* cnt_blk;    // per-block active counts to add up, or NULL
  int n_cnt_blk;
  int32_t* count_out;
  int32_t* count_out2;
  int32_t* nz_out;           // active neurons with h != 0, or NULL
  int32_t* tile_cnt;         // per column tile counters, zero at launch (the last block of a tile adds
                             // its partials), or NULL (partials only)
  const float* x_res;        // v_out = x_res + y
  float* y_out;              // y, or NULL
  float* v_out;              // or NULL
};

template <int WT, int TWC, bool EXPL>
void launch_k3_t(const pi_layer* L, const K3Shape& sh, const K3Args& a, hipStream_t st) {
  const int nblk = sh.ct * sh.nc;
  const int xcd = (nblk % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((k_down<WT, TWC, EXPL>), dim3(nblk), dim3(K3_WAVES * WAVE), 0, st, L->downT.w,
                     L->downT.scale, L->ffn, L->d, sh.ct, sh.nc, xcd, a.pid, a.ph, a.cap, a.idx, a.count, a.h_list,
                     L->b_down, a.y_part, a.cnt_blk, a.n_cnt_blk, a.count_out, a.count_out2, a.nz_out, a.tile_cnt,
                     a.x_res, a.y_out, a.v_out);
}

template <int WT, bool EXPL>
void launch_k3_w(const pi_layer* L, const K3Shape& sh, const K3Args& a, hipStream_t st) {
  switch (sh.twc) {
    case 1: return launch_k3_t<WT, 1, EXPL>(L, sh, a, st);
    case 2: return launch_k3_t<WT, 2, EXPL>(L, sh, a, st);
    case 4: return launch_k3_t<WT, 4, EXPL>(L, sh, a, st);
    default: return launch_k3_t<WT, 8, EXPL>(L, sh, a, st);
  }
}

// returns the number of partial vectors written
template <bool EXPL>
int k3(const pi_layer* L, const K3Args& a, hipStream_t st) {
  const K3Shape sh = k3_shape(L->d, L->w_dtype);
  switch (L->w_dtype) {
    case PI_F32: launch_k3_w<DT_F32, EXPL>(L, sh, a, st); break;
    case PI_F16: launch_k3_w<DT_F16, EXPL>(L, sh, a, st); break;
    default: launch_k3_w<DT_Q4, EXPL>(L, sh, a, st); break;
  }
  return sh.nc;
}

template <int WT, int ACT, int WCH>
void launch_up_list_w(const pi_layer* L, const float* x, const int32_t* idx, const int32_t* count, float* h_list,
                      hipStream_t st) {
  const int nb = std::max(1, std::min(1024, cdiv(L->ffn, 4)));
  hipLaunchKernelGGL((k_up_list<WT, ACT, WCH>), dim3(nb), dim3(kThreads), sizeof(float) * q4t_len(L->d), st, L->gate.w,
                     L->gate.scale, L->up.w, L->up.scale, L->bias, x, L->d, L->ffn, idx, count, h_list);
}

// chunks per lane per gathered up/gate row held at once (explicit lists)
constexpr int kWchF32[] = {2, 8};
constexpr int kWchF16[] = {2, 8, 14, 16};
constexpr int kWchQ4[] = {1, 6};
int up_list_wch(const pi_layer* L) {
  const int n = chunks_of(L->d, L->w_dtype);
  return L->w_dtype == PI_F32 ? pick(kWchF32, n) : L->w_dtype == PI_F16 ? pick(kWchF16, n) : pick(kWchQ4, n);
}

template <int WT, int ACT>
void launch_up_list_t(const pi_layer* L, const float* x, const int32_t* idx, const int32_t* count, float* h_list,
                      hipStream_t st) {
  const int wch = up_list_wch(L);
  if constexpr (WT == DT_F32) {
    if (wch == 2) return launch_up_list_w<WT, ACT, 2>(L, x, idx, count, h_list, st);
    return launch_up_list_w<WT, ACT, 8>(L, x, idx, count, h_list, st);
  } else if constexpr (WT == DT_F16) {
    if (wch == 2) return launch_up_list_w<WT, ACT, 2>(L, x, idx, count, h_list, st);
    if (wch == 8) return launch_up_list_w<WT, ACT, 8>(L, x, idx, count, h_list, st);
    if (wch == 14) return launch_up_list_w<WT, ACT, 14>(L, x, idx, count, h_list, st);
    return launch_up_list_w<WT, ACT, 16>(L, x, idx, count, h_list, st);
  } else {
    if (wch == 1) return launch_up_list_w<WT, ACT, 1>(L, x, idx, count, h_list, st);
    return launch_up_list_w<WT, ACT, 6>(L, x, idx, count, h_list, st);
  }
}

template <int WT>
void up_list_w(const pi_layer* L, const float* x, const int32_t* idx, const int32_t* count, float* h_list,
               hipStream_t st) {
  switch (L->act) {
    case PI_REGLU: return launch_up_list_t<WT, ACT_REGLU>(L, x, idx, count, h_list, st);
    case PI_RELU2: return launch_up_list_t<WT, ACT_RELU2>(L, x, idx, count, h_list, st);
    default: return launch_up_list_t<WT, ACT_RELU>(L, x, idx, count, h_list, st);
  }
}

void up_list(const pi_layer* L, const float* x, const int32_t* idx, const int32_t* count, float* h_list,
             hipStream_t st) {
  switch (L->w_dtype) {
    case PI_F32: return up_list_w<DT_F32>(L, x, idx, count, h_list, st);
    case PI_F16: return up_list_w<DT_F16>(L, x, idx, count, h_list, st);
    default: return up_list_w<DT_Q4>(L, x, idx, count, h_list, st);
  }
}

// ----------------------------------------------------------- batched path
// K splits of the first predictor GEMM so that the grid has ~256 blocks.
int bksplit(int r) { return std::max(1, std::min(kMaxKSplit, cdiv(256, cdiv(r, kBatchM)))); }

// x' of every sequence (glue of x_prev and y_prev, or x_prev itself when
// y_prev is NULL) to x_out / x_trace and as fp16 hi/lo operands.
void b_glue(const float* x_prev, const float* y_prev, int batch, int d, float* x_out, float* x_trace, const Ws& W,
            hipStream_t st) {
  const int bgv = d <= 4096 ? 1 : d <= 8192 ? 2 : 4;
  if (bgv == 1)
    hipLaunchKernelGGL(pib::k_bglue<1>, dim3(kBatchM), dim3(pib::BG_T), 0, st, x_prev, y_prev,
                     y_prev ? pib::bd_splits(d) : 0, batch, d, x_out, x_trace, W.xh, W.xl, W.sx, W.hmax);
  else if (bgv == 2)
    hipLaunchKernelGGL(pib::k_bglue<2>, dim3(kBatchM), dim3(pib::BG_T), 0, st, x_prev, y_prev,
                     y_prev ? pib::bd_splits(d) : 0, batch, d, x_out, x_trace, W.xh, W.xl, W.sx, W.hmax);
  else
    hipLaunchKernelGGL(pib::k_bglue<4>, dim3(kBatchM), dim3(pib::BG_T), 0, st, x_prev, y_prev,
                     y_prev ? pib::bd_splits(d) : 0, batch, d, x_out, x_trace, W.xh, W.xl, W.sx, W.hmax);
}

// per-sequence scores and masks, the union and its ascending list
// events[i] of a trace record, if it asks for one.  Under stream capture an
// event-record node is appended to the graph being captured (after the
// stream's current capture dependencies, which it then replaces), so that
// every replay stamps the event; otherwise the event is recorded on the stream.
void mark(const pi_trace* tr, int i, hipStream_t st) {
  if (!tr || !tr->events || i >= tr->n_events || !tr->events[i]) return;
  hipEvent_t ev = static_cast<hipEvent_t>(tr->events[i]);
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipGraph_t g = nullptr;
  const hipGraphNode_t* deps = nullptr;
  size_t nd = 0;
  if (hipStreamGetCaptureInfo_v2(st, &cs, nullptr, &g, &deps, &nd) != hipSuccess) return;  // error stays pending
  if (cs == hipStreamCaptureStatusActive) {
    hipGraphNode_t node = nullptr;
    if (hipGraphAddEventRecordNode(&node, g, deps, nd, ev) == hipSuccess)
      (void)hipStreamUpdateCaptureDependencies(st, &node, 1, hipStreamSetCaptureDependencies);
    return;
  }
  (void)hipEventRecord(ev, st);
}

void b_predict(const pi_layer* L, int batch, const Ws& W, float* scores, uint8_t* mask_out, int32_t* ulist,
               int32_t* ucount, int32_t* ucount2, int32_t* ucount3, hipStream_t st, const pi_trace* tr = nullptr) {
  const int ks = bksplit(L->rank);
  const dim3 g1(cdiv(L->rank, kBatchM) * ks);
  if (L->p_dtype == PI_F16)
    hipLaunchKernelGGL(pib::k_bpred1<DT_F16>, g1, dim3(256), 0, st, L->A, L->rank, L->d, ks, W.xh, W.xl, W.tpart);
  else
    hipLaunchKernelGGL(pib::k_bpred1<DT_F32>, g1, dim3(256), 0, st, L->A, L->rank, L->d, ks, W.xh, W.xl, W.tpart);
  mark(tr, 2, st);
  hipLaunchKernelGGL(pib::k_bsplit_t, dim3(kBatchM), dim3(pib::BT_T), 0, st, W.tpart, ks, L->rank, W.sx, W.th, W.tl,
                     W.st);
  mark(tr, 3, st);
  // T 32-neuron tiles per block (t read once per 32 T neurons): the T of 4, 3, 2, 1
  // whose blocks spread most evenly over the compute units, the larger on a tie
  // (the time is about rounds of 256 blocks times T)
  const float* pb = L->pbias ? L->pbias : L->bias;
  int nt = 4, best = 1 << 30;
  for (int t : {4, 3, 2, 1}) {
    const int cost = cdiv(cdiv(L->ffn, t * kBatchM), 256) * t;
    if (cost < best) { best = cost; nt = t; }
  }
  const dim3 g2(cdiv(L->ffn, nt * kBatchM));
#define PI_BSCORE(PT, NT)                                                                                      \
  hipLaunchKernelGGL((pib::k_bscore<PT, NT>), g2, dim3(256), 0, st, L->B, pb, L->ffn, L->rank, batch, W.th, W.tl, \
                     W.st, W.mnm, W.mask, W.cnt, scores, mask_out, L->hot)
#define PI_BSCORE_T(PT)                                                                                         \
  switch (nt) {                                                                                                 \
    case 4: PI_BSCORE(PT, 4); break;                                                                            \
    case 3: PI_BSCORE(PT, 3); break;                                                                            \
    case 2: PI_BSCORE(PT, 2); break;                                                                            \
    default: PI_BSCORE(PT, 1); break;                                                                           \
  }
  if (L->p_dtype == PI_F16) {
    PI_BSCORE_T(DT_F16)
  } else {
    PI_BSCORE_T(DT_F32)
  }
#undef PI_BSCORE_T
#undef PI_BSCORE
  mark(tr, 4, st);
  // the union list from the score kernel's union bytes and per-tile counts (multi-block, no atomics)
  hipLaunchKernelGGL(pib::k_bcompact, dim3(cdiv(bscore_blocks(L->ffn), 256)), dim3(256), 0, st, W.mask, W.cnt,
                     L->ffn, ulist, ucount, ucount2, ucount3);
  mark(tr, 5, st);
}

// The union size from which the batched FFN runs over every neuron.
int dense_min(const pi_layer* L) {
  const float fr = (L->dense_frac > 0.f) ? L->dense_frac : PI_DENSE_FRAC_DEFAULT;   // NaN: the default
  if (fr > 1.f) return L->ffn + 1;
  return std::max(1, (int)std::ceil((double)fr * L->ffn));
}

template <int WT, int ACT>
void b_ffn_t(const pi_layer* L, int batch, const Ws& W, const int32_t* ulist, const int32_t* ucount, float* y,
             hipStream_t st, const pi_trace* tr) {
  if constexpr (WT != DT_Q4) {
    hipLaunchKernelGGL((pib::k_bup<WT, ACT>), dim3(std::min(cdiv(L->ffn, kBatchM), kUpGrid)), dim3(pib::bup_waves(act_nmat<ACT>()) * WAVE),
                       0, st,
                       L->gate.w, L->gate.scale, L->up.w, L->up.scale, L->bias, L->ffn, L->d, W.xh, W.xl, ulist,
                       ucount, W.mnm, W.sx, W.h32, W.hmax, dense_min(L));
  } else {
    // Q4_0: K-split up GEMM on the batch operand staged in LDS, then the splits' sum and the
    // activation (for fp16 weights the one-pass GEMM over the whole K measured faster)
    const int ks = pib::bu_ks(L->d);
    const int groups = cdiv(cdiv(L->ffn, kBatchM), pib::BU_TPB);
    hipLaunchKernelGGL((pib::k_bup2<WT, act_nmat<ACT>()>), dim3(std::min(groups * ks, kUpGrid)), dim3(512), 0, st,
                       L->gate.w,
                       L->gate.scale, L->up.w, L->up.scale, L->ffn, L->d, ks, W.xh, W.xl, ulist, ucount, dense_min(L),
                       W.zpart);
    hipLaunchKernelGGL((pib::k_bup_epi<ACT>), dim3(std::min(cdiv(L->ffn, 256 / kBatchM), 2 * kUpGrid)), dim3(256), 0,
                       st, W.zpart, ks,
                       L->ffn, ulist, ucount, dense_min(L), L->bias, W.mnm, W.sx, W.h32, W.hmax);
  }
  mark(tr, 6, st);
  if constexpr (WT == DT_Q4)
    hipLaunchKernelGGL(pib::k_bdown_q4, dim3(cdiv(L->d, pib::BD_COLS) * pib::bd_splits(L->d)), dim3(512), 0, st,
                       static_cast<const uint8_t*>(L->downT.w), L->downT.scale, L->ffn, L->d, ulist, ucount, W.h32,
                       W.hmax, L->b_down, batch, y, dense_min(L), pib::bd_splits(L->d));
  else if constexpr (WT == DT_F16)
    hipLaunchKernelGGL(pib::k_bdown_f16, dim3(cdiv(L->d, pib::BD_COLS) * pib::bd_splits(L->d)), dim3(512), 0, st,
                       static_cast<const uint16_t*>(L->downT.w), L->ffn, L->d, ulist, ucount, W.h32, W.hmax,
                       L->b_down, batch, y, dense_min(L), pib::bd_splits(L->d));
  else
    hipLaunchKernelGGL(pib::k_bdown<WT>, dim3(cdiv(L->d, pib::BD_COLS) * pib::bd_splits(L->d)), dim3(512), 0, st,
                       L->downT.w, L->ffn, L->d, ulist, ucount, W.h32, W.hmax, L->b_down, batch, y, dense_min(L),
                       pib::bd_splits(L->d));
  mark(tr, 7, st);
}

// the FFN over the union list for every sequence: bd_splits(d) partial vectors
// y_part [bd_splits(d)][32][d] (rows b < batch written)
template <int WT>
void b_ffn_w(const pi_layer* L, int batch, const Ws& W, const int32_t* ulist, const int32_t* ucount, float* y,
             hipStream_t st, const pi_trace* tr) {
  switch (L->act) {
    case PI_REGLU: return b_ffn_t<WT, ACT_REGLU>(L, batch, W, ulist, ucount, y, st, tr);
    case PI_RELU2: return b_ffn_t<WT, ACT_RELU2>(L, batch, W, ulist, ucount, y, st, tr);
    default: return b_ffn_t<WT, ACT_RELU>(L, batch, W, ulist, ucount, y, st, tr);
  }
}

void b_ffn(const pi_layer* L, int batch, const Ws& W, const int32_t* ulist, const int32_t* ucount, float* y,
           hipStream_t st, const pi_trace* tr = nullptr) {
  switch (L->w_dtype) {
    case PI_F32: return b_ffn_w<DT_F32>(L, batch, W, ulist, ucount, y, st, tr);
    case PI_F16: return b_ffn_w<DT_F16>(L, batch, W, ulist, ucount, y, st, tr);
    default: return b_ffn_w<DT_Q4>(L, batch, W, ulist, ucount, y, st, tr);
  }
}

thread_local hipError_t g_last_hip = hipSuccess;   // behind this thread's last PI_EHIP

pi_status launch_status() {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return PI_OK;
  g_last_hip = e;
  return PI_EHIP;
}

}  // namespace

namespace {

// Host-only validation of a stack call; on success *WL is its workspace layout.
pi_status validate_stack(const pi_layer* layers, int32_t n_layers, const float* x, int32_t batch, const float* out,
                         const pi_trace* trace, WsLayout* WL) {
  if (!layers || n_layers <= 0) return PI_EINVAL;
  pi_status s;
  for (int l = 0; l < n_layers; ++l)
    if ((s = check_layer(&layers[l])) != PI_OK) return s;
  if ((s = check_batch(batch)) != PI_OK) return s;
  for (int l = 0; l < n_layers; ++l)
    if ((s = check_batched_ffn(&layers[l], batch)) != PI_OK) return s;
  if (!x || !aligned(x, 16) || !out) return PI_EINVAL;
  if (trace)
    for (int l = 0; l < n_layers; ++l)
      if (trace[l].mask && !aligned(trace[l].mask, 16)) return PI_EINVAL;
  Dims D;
  if (!dims_of(layers, n_layers, &D)) return PI_EINVAL;
  *WL = layout(D, batch);
  return PI_OK;
}

// Enqueue a validated stack call on stream st with workspace ws (WL.total bytes).
pi_status run_stack(const pi_layer* layers, int32_t n_layers, const float* x, int32_t batch, float* out,
                    int32_t* counts, int32_t* nz_counts, const pi_trace* trace, const WsLayout& WL, void* ws,
                    hipStream_t st) {
  Dims D;
  dims_of(layers, n_layers, &D);
  Ws W = carve(ws, WL);
  (void)hipGetLastError();
  if (batch > 1) {
    for (int l = 0; l < n_layers; ++l) {
      const pi_layer* L = &layers[l];
      const pi_trace* tr = trace ? &trace[l] : nullptr;
      const int cur = l & 1, prv = cur ^ 1;
      mark(tr, 0, st);
      b_glue(l == 0 ? x : W.x[prv], l == 0 ? nullptr : W.y[prv], batch, L->d, W.x[cur], tr ? tr->x_in : nullptr,
             W, st);
      mark(tr, 1, st);
      b_predict(L, batch, W, tr ? tr->scores : nullptr, tr ? tr->mask : nullptr, W.ulist, W.misc,
                counts ? counts + l : nullptr, nz_counts ? nz_counts + l : nullptr, st, tr);
      if (tr && (tr->idx || tr->count))   // the union list and count for the record
        hipLaunchKernelGGL(k_compact, dim3(1), dim3(1024), 0, st, W.mask, L->ffn, tr->idx ? tr->idx : W.ulist,
                           tr->count ? tr->count : W.misc + 1, nullptr, nullptr);
      b_ffn(L, batch, W, W.ulist, W.misc, W.y[cur], st, tr);
      if (tr && tr->y)   // the layer's y for the record: its partial vectors added in order
        hipLaunchKernelGGL(pib::k_bsum_y, dim3(cdiv(batch * L->d, 256)), dim3(256), 0, st, W.y[cur],
                           pib::bd_splits(L->d), batch, L->d,
                           tr->y);
    }
    const int last = (n_layers - 1) & 1;
    hipLaunchKernelGGL(pib::k_bglue_out, dim3(batch), dim3(pib::BG_T), 0, st, W.x[last], W.y[last],
                       pib::bd_splits(D.d), D.d, out);
    return launch_status();
  }
  for (int l = 0; l < n_layers; ++l) {
    const pi_layer* L = &layers[l];
    const pi_trace* tr = trace ? &trace[l] : nullptr;
    const int cur = l & 1;
    // v: the stack's input, then the previous layer's x' + y (written by its down projection)
    const bool glue = l > 0;
    const float* v = glue ? W.v : x;
    mark(tr, 0, st);
    k1(L, K1Args{v, glue, W.ss, W.t, W.tcnt, kMaxTiles}, st);
    mark(tr, 1, st);
    // the predictor's own mask goes to the record, or to W.pmask when only the
    // record's list asks for it
    uint8_t* pmask = tr ? (tr->mask ? tr->mask : (tr->idx ? W.pmask : nullptr)) : nullptr;
    k2(L, true, K2Args{W.t, glue ? W.ss : nullptr, v, W.x[cur], tr ? tr->x_in : nullptr,
                       tr ? tr->scores : nullptr, pmask, W.cnt, W.pid, W.ph}, st);
    mark(tr, 2, st);
    int32_t* c1 = counts ? counts + l : nullptr;
    int32_t* c2 = (tr && tr->count && !tr->idx) ? tr->count : nullptr;
    if (tr && tr->idx)   // ascending list of the predictor's mask, for the record
      hipLaunchKernelGGL(k_compact, dim3(1), dim3(1024), 0, st, pmask, L->ffn, tr->idx,
                         tr->count ? tr->count : W.misc, nullptr, nullptr);
    k3<false>(L, K3Args{W.pid, W.ph, k2_cap(L->ffn), nullptr, nullptr, nullptr, W.y[0], W.cnt, k2_blocks(L), c1, c2,
                        nz_counts ? nz_counts + l : nullptr, W.tcnt, W.x[cur], tr ? tr->y : nullptr, W.v},
              st);
    mark(tr, 3, st);
  }
  // out = glue(x' + y) of the last layer
  hipLaunchKernelGGL(k_glue_out, dim3(1), dim3(256), sizeof(float) * D.d, st, W.v, nullptr, 0, out, D.d);
  return launch_status();
}

}  // namespace

// ------------------------------------------------- workspace without allocation
// The workspace of pi_ffn_stack_static: one file-scope array, of which every
// GPU holds its own copy until the process ends.  In host code `scratch` names
// a host-side stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is ever passed
// to a kernel.
static __device__ __align__(256) unsigned char scratch[PI_STATIC_WORKSPACE_BYTES];

namespace {

constexpr size_t kStaticWsBytes = size_t(PI_STATIC_WORKSPACE_BYTES);
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on its first use).
pi_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_hip = e;
    return PI_EHIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return PI_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      g_last_hip = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return PI_EHIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PI_OK;
}

}  // namespace

extern "C" {

int32_t pi_abi_version(void) { return PI_ABI_VERSION; }

const char* pi_last_hip_error(void) { return hipGetErrorString(g_last_hip); }

const char* pi_status_str(pi_status s) {
  switch (s) {
    case PI_OK: return "ok";
    case PI_EINVAL: return "invalid argument";
    case PI_EUNSUPPORTED: return "unsupported";
    case PI_EWORKSPACE: return "workspace too small";
    case PI_EHIP: return "HIP launch error";
  }
  return "unknown status";
}

size_t pi_workspace_bytes(const pi_layer* layers, int32_t n_layers, int32_t batch) {
  Dims D;
  if (batch < 1 || batch > 32 || !dims_of(layers, n_layers, &D)) return 0;
  return layout(D, batch).total;
}

pi_status pi_predict(const pi_layer* layer, const float* x, int32_t batch, float* scores, uint8_t* mask,
                     int32_t* idx, int32_t* count, void* ws, size_t ws_bytes, void* stream) {
  pi_status s;
  if ((s = check_layer(layer)) != PI_OK) return s;
  if ((s = check_batch(batch)) != PI_OK) return s;
  if (!x || !aligned(x, 16) || !idx || !count) return PI_EINVAL;
  if (batch > 1 && !mask) return PI_EINVAL;
  Dims D;
  dims_of(layer, 1, &D);                 // the layer is valid (checked above)
  const WsLayout WL = layout(D, batch);
  if (!ws || ws_bytes < WL.total || !aligned(ws, kAlign)) return PI_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Ws W = carve(ws, WL);
  (void)hipGetLastError();
  if (batch > 1) {
    b_glue(x, nullptr, batch, layer->d, nullptr, nullptr, W, st);
    b_predict(layer, batch, W, scores, mask, idx, count, nullptr, nullptr, st);
    return launch_status();
  }
  k1(layer, K1Args{x, false, W.ss, W.t, nullptr, 0}, st);
  uint8_t* pm = mask ? mask : W.mask;
  k2(layer, false, K2Args{W.t, nullptr, nullptr, nullptr, nullptr, scores, pm, nullptr, nullptr, nullptr}, st);
  hipLaunchKernelGGL(k_compact, dim3(1), dim3(1024), 0, st, pm, layer->ffn, idx, count, nullptr, nullptr);
  return launch_status();
}

pi_status pi_sparse_ffn(const pi_layer* layer, const float* x, int32_t batch, const int32_t* idx,
                        const int32_t* count, const uint8_t* mask, float* y, void* ws, size_t ws_bytes,
                        void* stream) {
  pi_status s;
  if ((s = check_layer(layer)) != PI_OK) return s;
  if ((s = check_batch(batch)) != PI_OK) return s;
  if ((s = check_batched_ffn(layer, batch)) != PI_OK) return s;
  if (!x || !aligned(x, 16) || !idx || !count || !y) return PI_EINVAL;
  if ((batch == 1) != (mask == nullptr)) return PI_EINVAL;
  Dims D;
  dims_of(layer, 1, &D);                 // the layer is valid (checked above)
  const WsLayout WL = layout(D, batch);
  if (!ws || ws_bytes < WL.total || !aligned(ws, kAlign)) return PI_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Ws W = carve(ws, WL);
  (void)hipGetLastError();
  if (batch > 1) {
    // the listed neurons become the union (ascending, each once) with the caller's per-sequence masks
    b_glue(x, nullptr, batch, layer->d, nullptr, nullptr, W, st);
    hipLaunchKernelGGL(pib::k_bclear, dim3(cdiv(layer->ffn, 256)), dim3(256), 0, st, W.mask, W.mnm, layer->ffn);
    hipLaunchKernelGGL(pib::k_blist, dim3(cdiv(layer->ffn, 256)), dim3(256), 0, st, idx, count, layer->ffn, mask,
                       batch, W.mask, W.mnm);
    hipLaunchKernelGGL(k_compact, dim3(1), dim3(1024), 0, st, W.mask, layer->ffn, W.ulist, W.misc, nullptr, nullptr);
    b_ffn(layer, batch, W, W.ulist, W.misc, W.y[0], st);
    hipLaunchKernelGGL(pib::k_bsum_y, dim3(cdiv(batch * layer->d, 256)), dim3(256), 0, st, W.y[0],
                       pib::bd_splits(layer->d), batch, layer->d,
                       y);
    return launch_status();
  }
  up_list(layer, x, idx, count, W.h, st);
  const int np = k3<true>(layer, K3Args{nullptr, nullptr, 0, idx, count, W.h, W.y[0], nullptr, 0, nullptr, nullptr,
                                        nullptr},
                          st);
  hipLaunchKernelGGL(k_finalize, dim3(cdiv(layer->d, 256)), dim3(256), 0, st, W.y[0], np, y, layer->d);
  return launch_status();
}

pi_status pi_ffn_stack(const pi_layer* layers, int32_t n_layers, const float* x, int32_t batch, float* out,
                       int32_t* counts, int32_t* nz_counts, const pi_trace* trace, void* ws, size_t ws_bytes,
                       void* stream) {
  WsLayout WL;
  const pi_status s = validate_stack(layers, n_layers, x, batch, out, trace, &WL);
  if (s != PI_OK) return s;
  if (!ws || ws_bytes < WL.total || !aligned(ws, kAlign)) return PI_EWORKSPACE;
  return run_stack(layers, n_layers, x, batch, out, counts, nz_counts, trace, WL, ws,
                   static_cast<hipStream_t>(stream));
}

pi_status pi_ffn_stack_static(const pi_layer* layers, int32_t n_layers, const float* x, int32_t batch, float* out,
                              int32_t* counts, int32_t* nz_counts, const pi_trace* trace, void* stream) {
  WsLayout WL;
  const pi_status s = validate_stack(layers, n_layers, x, batch, out, trace, &WL);
  if (s != PI_OK) return s;
  if (WL.total > kStaticWsBytes) return PI_EWORKSPACE;   // checked before any HIP call
  void* ws = nullptr;
  const pi_status sp = scratch_of_current_device(&ws);
  if (sp != PI_OK) return sp;
  return run_stack(layers, n_layers, x, batch, out, counts, nz_counts, trace, WL, ws,
                   static_cast<hipStream_t>(stream));
}

}  // extern "C"
