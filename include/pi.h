/*
 * pi.h -- C ABI of the predictor-guided, neuron-aware sparse FFN for one AMD
 * Instinct MI355X (gfx950).
 *
 * The method (PowerInfer pages): for the current token, a per-layer low-rank
 * predictor marks which FFN neurons will fire, and only those neurons' rows of
 * the up/gate projections and columns of the down projection are read and
 * computed, with no conversion of the weights into a sparse format at run time
 * (unite.ai article, "Online-Phase", "Adaptive Sparsity-Prädiktoren",
 * "Neuronenbewusster Operator"; 机器之心 article, Fig. 8 paragraph; GeekNews
 * summary, "CPU/GPUハイブリッド推論方式").  Every neuron stays resident in HBM;
 * the hot/cold profile survives only as the storage order of the neurons.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    allocates nothing, keeps no pointer after it returns and never
 *    synchronises the stream.  `stream` is a hipStream_t passed as void*
 *    (NULL = the default stream).
 *  - Matrices are row-major.  Neurons are in STORAGE order (hot-first in the
 *    shipped workloads); lists and masks refer to storage slots.  A table that
 *    maps slots back to original neuron ids is the caller's business.
 *  - Validation is synchronous and host-only: PI_EINVAL / PI_EUNSUPPORTED /
 *    PI_EWORKSPACE are returned before anything is enqueued.  PI_EHIP means a
 *    launch was rejected (hipGetLastError); faults inside kernels surface at
 *    the caller's next synchronisation.
 *  - Rules checked: non-NULL required pointers; d, ffn, rank > 0;
 *    bias and pbias 16-byte aligned;
 *    d % 64 == 0; rank % 64 == 0; weight, predictor and activation pointers
 *    16-byte aligned, Q4_0 scales 4-byte aligned; 1 <= batch <= 32;
 *    act REGLU needs `gate`; predictor dtype F32 or F16 (Q4_0 predictor:
 *    PI_EUNSUPPORTED); d <= 16384 and rank <= 4096 (vectors are staged whole
 *    in LDS; larger: PI_EUNSUPPORTED); ffn <= 2^21 (the score kernel keeps
 *    each wave's active neurons in LDS) and, for the FFN at batch > 1,
 *    ffn <= 65536 (PI_EUNSUPPORTED otherwise); every layer of a stack has the
 *    same d.
 *  - Calls on distinct workspaces are independent; calls sharing a workspace
 *    must be ordered on one stream.
 *  - Batch 1 runs GEMV kernels over the active rows.  Batch 2..32 runs each
 *    sequence's predictor, takes the union of the masks (PowerInfer pages:
 *    batched decoding, 机器之心 article, Fig. 14 paragraph) and computes the
 *    FFN over the union's rows as gathered GEMMs on the matrix cores, with
 *    fp16 hi/lo splits of the activations so that results match fp32
 *    accumulation; a sequence's output equals its own batch-1 result (a
 *    neuron in the union but off in that sequence's mask contributes 0).
 */
#ifndef PI_H_
#define PI_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PI_ABI_VERSION 6

/* Union fraction at and above which the batched FFN runs over every neuron
 * when pi_layer.dense_frac is 0 (see pi_layer.dense_frac). */
#define PI_DENSE_FRAC_DEFAULT 0.9f

typedef enum {
  PI_OK = 0,
  PI_EINVAL = 1,        /* bad argument (NULL, size, alignment, dtype/act combination) */
  PI_EUNSUPPORTED = 2,  /* valid request the library does not implement */
  PI_EWORKSPACE = 3,    /* ws NULL or ws_bytes < pi_workspace_bytes(...) */
  PI_EHIP = 4           /* a kernel launch failed */
} pi_status;

typedef enum { PI_F32 = 0, PI_F16 = 1, PI_Q4_0 = 2 } pi_dtype;

/* ReLU: h = max(b + W_up x, 0).  ReGLU: h = max(b + W_gate x, 0) * (W_up x).
 * Squared ReLU: h = max(b + W_up x, 0)^2.
 * (GeekNews summary: ReLU / ReGLU / Squared-ReLU models.) */
typedef enum { PI_RELU = 0, PI_REGLU = 1, PI_RELU2 = 2 } pi_act;

/* One weight matrix [ffn][d].  F32/F16: `w` points at ffn*d elements and
 * `scale` is NULL.  Q4_0 (blocks of 32 4-bit values q in [0,15] with one
 * binary16 scale s, w = s*(q-8)): `w` points at nibbles uint8 [ffn][d/2] and
 * `scale` at binary16 bits [ffn][d/32].  Inside a 32-block, weight j < 16 is
 * the low nibble of byte j and weight j+16 the high nibble of byte j. */
typedef struct {
  const void* w;
  const uint16_t* scale;
} pi_mat;

/* One FFN layer with its predictor. */
typedef struct {
  int32_t d;        /* model width */
  int32_t ffn;      /* number of FFN neurons */
  int32_t rank;     /* predictor rank r */
  int32_t act;      /* pi_act */
  int32_t w_dtype;  /* pi_dtype of gate/up/downT */
  int32_t p_dtype;  /* pi_dtype of A and B (F32 or F16) */
  const void* A;    /* [rank][d] predictor first matrix */
  const void* B;    /* [ffn][rank] predictor second matrix, storage order */
  const float* bias;/* [ffn] bias of the gate (ReGLU) or up (ReLU, Squared ReLU) projection */
  const float* pbias;/* [ffn] predictor output bias, s_i = pbias_i + B[i] . (A x);
                       NULL = use `bias` */
  pi_mat gate;      /* [ffn][d]; REGLU only (ignored for RELU) */
  pi_mat up;        /* [ffn][d] */
  pi_mat downT;     /* [ffn][d]; row i is column i of W_down, so the down projection
                       over active neurons is a row gather too */
  const float* b_down; /* [d] or NULL */
  int32_t hot;      /* hot-dense prefix, 0 <= hot <= ffn (else PI_EINVAL): storage slots
                       [0, hot) -- the hottest neurons after the hot-first permutation --
                       are active for every token and sequence without a prediction (their
                       rows of B are never read, their scores are not written, their mask
                       bytes are 1); only the cold tail [hot, ffn) is predicted and
                       gathered.  0 = every neuron is predicted.  The on-GPU form of the
                       hot/cold neuron split (PowerInfer repository README, "hot-activated
                       neurons"; unite.ai article, "Neuronen-Platzierung und -Verwaltung";
                       机器之心 article, hot/cold neuron paragraph). */
  float dense_frac; /* batch > 1: when the union of the sequences' masks holds at least
                       dense_frac * ffn neurons, the up/gate and down GEMMs run over every
                       neuron in storage order instead of the gathered union rows (a
                       neuron outside the union gets h = 0, so the result is the same).
                       As the batch grows the union tends to every neuron (机器之心
                       article, Fig. 14 paragraph).  0 (or NaN) = the library's default
                       (PI_DENSE_FRAC_DEFAULT); a value above 1 = never. */
} pi_layer;

/* Optional per-layer record written by pi_ffn_stack (any field may be NULL). */
typedef struct {
  float* x_in;      /* [batch][d]   input of the layer */
  float* scores;    /* [batch][ffn] predictor scores */
  uint8_t* mask;    /* [batch][ffn] 1 if score > 0; 16-byte aligned (PI_EINVAL) */
  int32_t* idx;     /* [ffn]        ascending storage ids of the union mask */
  int32_t* count;   /* [1]          number of entries in idx */
  float* y;         /* [batch][d]   the layer's FFN output y_l (before the glue) */
  /* Timing: hipEvent_t handles (as void*) recorded on the stream, events[0]
   * before the layer's first kernel and events[i] after its i-th kernel, for
   * i < n_events.  Kernels of a layer, in order -- batch 1: predictor GEMV 1
   * with the glue, scores with the fused up/gate gather, down projection;
   * batch > 1: glue, predictor GEMM 1, its split sum, scores and union, union
   * compaction, up/gate GEMM (for Q4_0 weights its K-split GEMM and the
   * epilogue that adds the splits, as one interval), down GEMM.  Record-only kernels of the trace
   * (list compaction, the sum of y's partial vectors) are not counted. */
  void** events;
  int32_t n_events;
} pi_trace;

/* Workspace needed by any entry point for these layers at this batch.
 * Returns 0 if the layer array is invalid. */
size_t pi_workspace_bytes(const pi_layer* layers, int32_t n_layers, int32_t batch);

/*
 * pi_predict -- predictor, threshold and compaction for one layer
 * (unite.ai article, "Online-Phase": predict the activated neurons of the
 * current layer and skip the others; 机器之心 article, Fig. 8 paragraph).
 *   t = A x_b;  s_{b,i} = pbias_i + B[i] . t  (float32 accumulation; pbias
 *   defaults to bias)
 *   mask_{b,i} = (s_{b,i} > 0)  strict; zero and NaN are inactive
 *   idx = ascending storage ids i with mask_{b,i} = 1 for some b; *count = |idx|
 * x: [batch][d] float32.  scores: [batch][ffn] or NULL.  mask: [batch][ffn],
 * may be NULL when batch == 1 and is required when batch > 1 (PI_EINVAL).
 * idx: [ffn] int32.  count: [1] int32, written on the device (the host never
 * reads it inside the library).
 */
pi_status pi_predict(const pi_layer* layer, const float* x, int32_t batch, float* scores,
                     uint8_t* mask, int32_t* idx, int32_t* count, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * pi_sparse_ffn -- neuron-aware sparse FFN over a caller-supplied list
 * (unite.ai article, "Neuronenbewusster Operator": individual rows and columns
 * of the matrices, no sparse-format conversion).
 *   for each listed i (and, when batch > 1, only where mask_{b,i} = 1):
 *     ReLU:  h = max(bias_i + up[i] . x_b, 0)
 *     ReGLU: h = max(bias_i + gate[i] . x_b, 0) * (up[i] . x_b)
 *     Squared ReLU: h = max(bias_i + up[i] . x_b, 0)^2
 *   y_b = sum_i h * downT[i]  (+ b_down)
 * idx: ascending or not, distinct entries, first min(*count, ffn) used (count
 * is read on the device and clamped to [0, ffn]); entries outside [0, ffn)
 * are skipped.  mask: [batch][ffn] uint8, NULL iff batch == 1 (PI_EINVAL
 * otherwise).  y: [batch][d] float32, fully overwritten.
 */
pi_status pi_sparse_ffn(const pi_layer* layer, const float* x, int32_t batch, const int32_t* idx,
                        const int32_t* count, const uint8_t* mask, float* y, void* ws,
                        size_t ws_bytes, void* stream);

/*
 * pi_ffn_stack -- n_layers layers in sequence, each predict -> sparse FFN,
 * joined by a residual with a parameter-free RMS norm (not on the pages; it
 * keeps firing rates stable through the stack):
 *   x_0 = x;  x_{l+1} = v / sqrt(mean(v^2) + 1e-6),  v = x_l + y_l;  out = x_L
 * At batch 1 the down projection reads only the rows of the active neurons
 * whose h is nonzero (a zero term adds nothing to y; ReLU zeroes every
 * marked neuron whose pre-activation turns out <= 0).
 * counts: [n_layers] int32 active count per layer (union when batch > 1), or
 * NULL.  nz_counts: [n_layers] int32, or NULL: rows of downT read per layer
 * (batch 1: active neurons with h != 0; batch > 1: the union count).
 * trace: array of n_layers records, or NULL.
 */
pi_status pi_ffn_stack(const pi_layer* layers, int32_t n_layers, const float* x, int32_t batch,
                       float* out, int32_t* counts, int32_t* nz_counts, const pi_trace* trace,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * pi_ffn_stack_static -- pi_ffn_stack without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  It computes exactly what
 * pi_ffn_stack computes, with the same kernels, and calls no allocating
 * routine: its workspace is a file-scope device array of
 * PI_STATIC_WORKSPACE_BYTES that every GPU the library runs on holds until the
 * process ends (its device address is looked up once per device, on the
 * first call with that device current).
 * Returns PI_EWORKSPACE, before any HIP call, when
 * pi_workspace_bytes(layers, n_layers, batch) exceeds PI_STATIC_WORKSPACE_BYTES
 * (96 MiB covers batch 1 at every accepted shape, and batch 2..32 up to
 * d = 12288 with ffn = 49152 and rank = 1024 for every layer but ReGLU with
 * Q4_0 weights, which needs 135 MiB there).  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (other streams, other threads) race and give undefined
 * results; calls ordered on one stream are independent.
 */
#define PI_STATIC_WORKSPACE_BYTES (96u << 20)
pi_status pi_ffn_stack_static(const pi_layer* layers, int32_t n_layers, const float* x, int32_t batch,
                              float* out, int32_t* counts, int32_t* nz_counts, const pi_trace* trace,
                              void* stream);

const char* pi_status_str(pi_status s);
int32_t pi_abi_version(void);
/* Name of the HIP error behind the calling thread's most recent PI_EHIP
 * ("no error" before any).  Static string, not to be freed. */
const char* pi_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* PI_H_ */
