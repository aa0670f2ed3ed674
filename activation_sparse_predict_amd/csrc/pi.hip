// Host side of the C ABI declared in include/pi.h: argument validation,
// workspace layout, launch configuration and kernel dispatch.
#include "pi.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

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

pi_status check_layer(const pi_layer* L) {
  if (!L) return PI_EINVAL;
  if (L->d <= 0 || L->ffn <= 0 || L->rank <= 0) return PI_EINVAL;
  if (L->d % 64 != 0 || L->rank % 64 != 0) return PI_EINVAL;
  if (L->act != PI_RELU && L->act != PI_REGLU) return PI_EINVAL;
  if (L->w_dtype != PI_F32 && L->w_dtype != PI_F16 && L->w_dtype != PI_Q4_0) return PI_EINVAL;
  if (L->p_dtype == PI_Q4_0) return PI_EUNSUPPORTED;
  if (L->p_dtype != PI_F32 && L->p_dtype != PI_F16) return PI_EINVAL;
  if (!L->A || !L->B || !L->bias) return PI_EINVAL;
  if (!aligned(L->A, 16) || !aligned(L->B, 16) || !aligned(L->bias, 16)) return PI_EINVAL;
  pi_status s;
  if ((s = check_mat(L->up, L->w_dtype)) != PI_OK) return s;
  if ((s = check_mat(L->downT, L->w_dtype)) != PI_OK) return s;
  if (L->act == PI_REGLU && (s = check_mat(L->gate, L->w_dtype)) != PI_OK) return s;
  if (L->b_down && !aligned(L->b_down, 4)) return PI_EINVAL;
  if (L->pbias && !aligned(L->pbias, 16)) return PI_EINVAL;
  return PI_OK;
}

pi_status check_batch(int32_t batch) {
  if (batch < 1 || batch > 32) return PI_EINVAL;
  if (batch != 1) return PI_EUNSUPPORTED;
  return PI_OK;
}

// -------------------------------------------------------------- workspace
struct Dims {
  int d = 0, fmax = 0, rmax = 0;
};

struct WsLayout {
  size_t t, xbuf, ybuf, bits, h, misc, total;
};

WsLayout layout(const Dims& D, int batch) {
  WsLayout w{};
  size_t o = 0;
  w.t = o;    o += align_up(sizeof(float) * (size_t)D.rmax * batch);
  w.xbuf = o; o += align_up(sizeof(float) * (size_t)D.d * batch) * 2;
  w.ybuf = o; o += align_up(sizeof(double) * (size_t)D.d * batch) * 2;
  w.bits = o; o += align_up(sizeof(uint32_t) * (size_t)((D.fmax + 31) / 32) * batch);
  w.h = o;    o += align_up(sizeof(float) * (size_t)D.fmax * batch);
  w.misc = o; o += kAlign;
  w.total = o;
  return w;
}

struct Ws {
  float* t;
  float* x[2];
  double* y[2];
  uint32_t* bits;
  float* h;
  int32_t* misc;
};

Ws carve(void* base, const WsLayout& L, const Dims& D, int batch) {
  char* b = static_cast<char*>(base);
  Ws w;
  w.t = reinterpret_cast<float*>(b + L.t);
  const size_t xs = align_up(sizeof(float) * (size_t)D.d * batch);
  const size_t ys = align_up(sizeof(double) * (size_t)D.d * batch);
  w.x[0] = reinterpret_cast<float*>(b + L.xbuf);
  w.x[1] = reinterpret_cast<float*>(b + L.xbuf + xs);
  w.y[0] = reinterpret_cast<double*>(b + L.ybuf);
  w.y[1] = reinterpret_cast<double*>(b + L.ybuf + ys);
  w.bits = reinterpret_cast<uint32_t*>(b + L.bits);
  w.h = reinterpret_cast<float*>(b + L.h);
  w.misc = reinterpret_cast<int32_t*>(b + L.misc);
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
  }
  return true;
}

// ---------------------------------------------------------- launch shapes
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / WAVE;

int k1_blocks(int r) { return std::max(1, std::min(1024, (r + kWaves - 1) / kWaves)); }

int k2_blocks(int f) {
  int nb = std::min(f, 512);
  nb = std::max(nb, (f + K2_MAX_PER_BLOCK - 1) / K2_MAX_PER_BLOCK);
  return std::max(1, nb);
}

int epl_of(int dt) { return dt == PI_F32 ? 4 : (dt == PI_F16 ? 8 : 32); }

void k3_shape(int d, int dt, int* CT, int* NC) {
  const int tw = WAVE * epl_of(dt);
  *CT = (d + tw - 1) / tw;
  *NC = std::max(1, std::min(64, 256 / *CT));
}

// ---------------------------------------------------------------- dispatch
template <int PT>
void launch_k1(const pi_layer* L, const float* x_prev, const double* y_prev, float* x_out, float* x_trace,
               float* t, double* zero_y, int zero_y_n, uint32_t* zero_w, int zero_w_n, hipStream_t st) {
  const int nb = k1_blocks(L->rank);
  hipLaunchKernelGGL(k_predict_t<PT>, dim3(nb), dim3(kThreads), sizeof(float) * L->d, st, L->A, L->rank, L->d,
                     x_prev, y_prev, x_out, x_trace, t, zero_y, zero_y_n, zero_w, zero_w_n);
}

void k1(const pi_layer* L, const float* x_prev, const double* y_prev, float* x_out, float* x_trace, float* t,
        double* zero_y, int zero_y_n, uint32_t* zero_w, int zero_w_n, hipStream_t st) {
  if (L->p_dtype == PI_F32)
    launch_k1<DT_F32>(L, x_prev, y_prev, x_out, x_trace, t, zero_y, zero_y_n, zero_w, zero_w_n, st);
  else
    launch_k1<DT_F16>(L, x_prev, y_prev, x_out, x_trace, t, zero_y, zero_y_n, zero_w, zero_w_n, st);
}

template <int PT, int WT, int ACT, bool FUSE>
void launch_k2_t(const pi_layer* L, const float* t, const float* xcur, float* scores, uint8_t* mask,
                 uint32_t* bits, float* h, hipStream_t st) {
  const int nb = k2_blocks(L->ffn);
  const size_t lds = sizeof(float) * ((size_t)L->rank + (FUSE ? (size_t)L->d : 0));
  hipLaunchKernelGGL((k_score<PT, WT, ACT, FUSE>), dim3(nb), dim3(kThreads), lds, st, L->B,
                     L->pbias ? L->pbias : L->bias, L->bias, t, L->ffn,
                     L->rank, L->gate.w, L->gate.scale, L->up.w, L->up.scale, xcur, L->d, scores, mask, bits, h);
}

template <int PT, bool FUSE>
void launch_k2_w(const pi_layer* L, const float* t, const float* xcur, float* scores, uint8_t* mask,
                 uint32_t* bits, float* h, hipStream_t st) {
  const bool reglu = L->act == PI_REGLU;
  switch (L->w_dtype) {
    case PI_F32:
      reglu ? launch_k2_t<PT, DT_F32, ACT_REGLU, FUSE>(L, t, xcur, scores, mask, bits, h, st)
            : launch_k2_t<PT, DT_F32, ACT_RELU, FUSE>(L, t, xcur, scores, mask, bits, h, st);
      break;
    case PI_F16:
      reglu ? launch_k2_t<PT, DT_F16, ACT_REGLU, FUSE>(L, t, xcur, scores, mask, bits, h, st)
            : launch_k2_t<PT, DT_F16, ACT_RELU, FUSE>(L, t, xcur, scores, mask, bits, h, st);
      break;
    default:
      reglu ? launch_k2_t<PT, DT_Q4, ACT_REGLU, FUSE>(L, t, xcur, scores, mask, bits, h, st)
            : launch_k2_t<PT, DT_Q4, ACT_RELU, FUSE>(L, t, xcur, scores, mask, bits, h, st);
      break;
  }
}

void k2(const pi_layer* L, bool fuse_up, const float* t, const float* xcur, float* scores, uint8_t* mask,
        uint32_t* bits, float* h, hipStream_t st) {
  if (L->p_dtype == PI_F32) {
    fuse_up ? launch_k2_w<DT_F32, true>(L, t, xcur, scores, mask, bits, h, st)
            : launch_k2_w<DT_F32, false>(L, t, xcur, scores, mask, bits, h, st);
  } else {
    fuse_up ? launch_k2_w<DT_F16, true>(L, t, xcur, scores, mask, bits, h, st)
            : launch_k2_w<DT_F16, false>(L, t, xcur, scores, mask, bits, h, st);
  }
}

template <int WT, bool EXPL>
void launch_k3_t(const pi_layer* L, const uint32_t* bits, const float* h_full, const int32_t* idx,
                 const int32_t* count, const float* h_list, double* y_acc, int32_t* count_out, hipStream_t st) {
  int CT, NC;
  k3_shape(L->d, L->w_dtype, &CT, &NC);
  const size_t lds = sizeof(float) * kWaves * WAVE * Tr<WT>::EPL;
  hipLaunchKernelGGL((k_down<WT, EXPL>), dim3(CT * NC), dim3(kThreads), lds, st, L->downT.w, L->downT.scale,
                     L->ffn, L->d, CT, bits, h_full, idx, count, h_list, L->b_down, y_acc, count_out);
}

template <bool EXPL>
void k3(const pi_layer* L, const uint32_t* bits, const float* h_full, const int32_t* idx, const int32_t* count,
        const float* h_list, double* y_acc, int32_t* count_out, hipStream_t st) {
  switch (L->w_dtype) {
    case PI_F32: launch_k3_t<DT_F32, EXPL>(L, bits, h_full, idx, count, h_list, y_acc, count_out, st); break;
    case PI_F16: launch_k3_t<DT_F16, EXPL>(L, bits, h_full, idx, count, h_list, y_acc, count_out, st); break;
    default: launch_k3_t<DT_Q4, EXPL>(L, bits, h_full, idx, count, h_list, y_acc, count_out, st); break;
  }
}

template <int WT, int ACT>
void launch_up_list_t(const pi_layer* L, const float* x, const int32_t* idx, const int32_t* count, float* h_list,
                      double* y_acc, hipStream_t st) {
  const int nb = std::max(1, std::min(512, (L->ffn + kWaves - 1) / kWaves));
  hipLaunchKernelGGL((k_up_list<WT, ACT>), dim3(nb), dim3(kThreads), sizeof(float) * L->d, st, L->gate.w,
                     L->gate.scale, L->up.w, L->up.scale, L->bias, x, L->d, L->ffn, idx, count, h_list, y_acc);
}

void up_list(const pi_layer* L, const float* x, const int32_t* idx, const int32_t* count, float* h_list,
             double* y_acc, hipStream_t st) {
  const bool reglu = L->act == PI_REGLU;
  switch (L->w_dtype) {
    case PI_F32:
      reglu ? launch_up_list_t<DT_F32, ACT_REGLU>(L, x, idx, count, h_list, y_acc, st)
            : launch_up_list_t<DT_F32, ACT_RELU>(L, x, idx, count, h_list, y_acc, st);
      break;
    case PI_F16:
      reglu ? launch_up_list_t<DT_F16, ACT_REGLU>(L, x, idx, count, h_list, y_acc, st)
            : launch_up_list_t<DT_F16, ACT_RELU>(L, x, idx, count, h_list, y_acc, st);
      break;
    default:
      reglu ? launch_up_list_t<DT_Q4, ACT_REGLU>(L, x, idx, count, h_list, y_acc, st)
            : launch_up_list_t<DT_Q4, ACT_RELU>(L, x, idx, count, h_list, y_acc, st);
      break;
  }
}

pi_status launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? PI_OK : PI_EHIP;
}

}  // namespace

extern "C" {

int32_t pi_abi_version(void) { return PI_ABI_VERSION; }

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
  Dims D{layer->d, layer->ffn, layer->rank};
  const WsLayout WL = layout(D, batch);
  if (!ws || ws_bytes < WL.total || !aligned(ws, kAlign)) return PI_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Ws W = carve(ws, WL, D, batch);
  const int nwords = (layer->ffn + 31) / 32;
  (void)hipGetLastError();
  k1(layer, x, nullptr, nullptr, nullptr, W.t, nullptr, 0, W.bits, nwords, st);
  k2(layer, false, W.t, nullptr, scores, mask, W.bits, nullptr, st);
  hipLaunchKernelGGL(k_compact, dim3(1), dim3(1024), 0, st, W.bits, layer->ffn, idx, count);
  return launch_status();
}

pi_status pi_sparse_ffn(const pi_layer* layer, const float* x, int32_t batch, const int32_t* idx,
                        const int32_t* count, const uint8_t* mask, float* y, void* ws, size_t ws_bytes,
                        void* stream) {
  pi_status s;
  if ((s = check_layer(layer)) != PI_OK) return s;
  if ((s = check_batch(batch)) != PI_OK) return s;
  if (!x || !aligned(x, 16) || !idx || !count || !y) return PI_EINVAL;
  if (batch == 1 && mask) return PI_EINVAL;
  Dims D{layer->d, layer->ffn, layer->rank};
  const WsLayout WL = layout(D, batch);
  if (!ws || ws_bytes < WL.total || !aligned(ws, kAlign)) return PI_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Ws W = carve(ws, WL, D, batch);
  (void)hipGetLastError();
  up_list(layer, x, idx, count, W.h, W.y[0], st);
  k3<true>(layer, nullptr, nullptr, idx, count, W.h, W.y[0], nullptr, st);
  hipLaunchKernelGGL(k_finalize, dim3((layer->d + 255) / 256), dim3(256), 0, st, W.y[0], y, layer->d);
  return launch_status();
}

pi_status pi_ffn_stack(const pi_layer* layers, int32_t n_layers, const float* x, int32_t batch, float* out,
                       int32_t* counts, const pi_trace* trace, void* ws, size_t ws_bytes, void* stream) {
  if (!layers || n_layers <= 0) return PI_EINVAL;
  pi_status s;
  for (int l = 0; l < n_layers; ++l)
    if ((s = check_layer(&layers[l])) != PI_OK) return s;
  if ((s = check_batch(batch)) != PI_OK) return s;
  if (!x || !aligned(x, 16) || !out) return PI_EINVAL;
  Dims D;
  if (!dims_of(layers, n_layers, &D)) return PI_EINVAL;
  const WsLayout WL = layout(D, batch);
  if (!ws || ws_bytes < WL.total || !aligned(ws, kAlign)) return PI_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Ws W = carve(ws, WL, D, batch);
  (void)hipGetLastError();
  for (int l = 0; l < n_layers; ++l) {
    const pi_layer* L = &layers[l];
    const pi_trace* tr = trace ? &trace[l] : nullptr;
    const int cur = l & 1, prv = cur ^ 1;
    const float* x_prev = l == 0 ? x : W.x[prv];
    const double* y_prev = l == 0 ? nullptr : W.y[prv];
    const int nwords = (L->ffn + 31) / 32;
    k1(L, x_prev, y_prev, W.x[cur], tr ? tr->x_in : nullptr, W.t, W.y[cur], L->d, W.bits, nwords, st);
    k2(L, true, W.t, W.x[cur], tr ? tr->scores : nullptr, tr ? tr->mask : nullptr, W.bits, W.h, st);
    if (tr && tr->idx) {
      // list for the record only; the down projection reads the mask bits directly
      hipLaunchKernelGGL(k_compact, dim3(1), dim3(1024), 0, st, W.bits, L->ffn, tr->idx,
                         tr->count ? tr->count : W.misc);
    }
    const bool tr_cnt = tr && tr->count && !tr->idx;   // count record without a list
    int32_t* cnt_out = counts ? counts + l : (tr_cnt ? tr->count : nullptr);
    k3<false>(L, W.bits, W.h, nullptr, nullptr, nullptr, W.y[cur], cnt_out, st);
    if (counts && tr_cnt) hipLaunchKernelGGL(k_copy_i32, dim3(1), dim3(64), 0, st, counts + l, tr->count, 1);
  }
  {
    const int last = (n_layers - 1) & 1;
    hipLaunchKernelGGL(k_glue_out, dim3(1), dim3(256), sizeof(float) * D.d, st, W.x[last], W.y[last], out, D.d);
  }
  return launch_status();
}

}  // extern "C"
