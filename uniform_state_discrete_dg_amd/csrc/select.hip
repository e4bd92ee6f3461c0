// select.hip -- the integer end of a denoising step: canvas initialisation,
// the entropy-bounded accept walk, re-noise and the adaptive-stop flags.
// One workgroup of 256 threads handles the whole canvas (N <= 256).
//
// [P3] §5.4: positions are ordered from lowest to highest entropy and walked
// in that order; a position is accepted while the running sum of entropies
// (less their maximum, which in ascending order is the current one) stays
// within the threshold, and the first failure ends the walk.  [P5] states
// the plain running sum (rule CUMSUM).  Every rejected position is
// re-noised with a fresh uniform token; accepted ones take the candidate.
// [P3] §5.3 / [P5] adaptive stop: the flags say whether every entropy is
// below the confidence threshold and count the steps in a row whose
// predictions (or, by the configured rule, the canvas) did not change.
// Masked sampler ([P1] §1, [P3] §3.1): only positions holding [MASK] are
// walked, rejected ones keep [MASK] and decided ones are never revisited.
//
// The walk is evaluated in parallel: each position's key (entropy bits << 32
// | position; unique, so the order is total) is sorted ascending by a
// bitonic network over the workgroup's 256 threads, each ranked entropy is
// turned into 2^-32-nat fixed point and prefix-summed in 64-bit integers
// (exact, so independent of summation order), and a rank is accepted iff its
// prefix test holds: the tests are monotone in the rank, so this equals the
// sequential walk with its first failure ending it.
#include "dg_device.h"
#include "dg_kernels.h"
#include "dgdenoise.h"

namespace dg {

__global__ void canvas_init_kernel(int32_t *tokens, int32_t *status, int N, int log2v, uint64_t seed,
                                   uint32_t canvas_id, int mask_id) {
  const int i = threadIdx.x + blockIdx.x * blockDim.x;
  if (i < N) tokens[i] = mask_id >= 0 ? mask_id : uniform_token(seed, (uint32_t)i, 0u, canvas_id, 0u, log2v);
  if (i < DG_STATUS_WORDS)
    status[i] = (i == DG_ST_STEP) ? -1 : (i == DG_ST_MASKED) ? (mask_id >= 0 ? N : -1) : 0;
}

hipError_t canvas_init(int32_t *tokens, int32_t *status, int N, int log2v, uint64_t seed,
                       uint32_t canvas_id, int mask_id, hipStream_t s) {
  hipLaunchKernelGGL(canvas_init_kernel, dim3(1), dim3(256), 0, s, tokens, status, N, log2v, seed, canvas_id,
                     mask_id);
  return hipGetLastError();
}

// pred: each position's prediction (the most likely token, as the int bits
// of top[i].x); pred_prev: the previous step's, replaced by this step's.
__device__ __forceinline__ void select_body(const float *__restrict__ entropy, const int32_t *__restrict__ argmax,
                                            int32_t *__restrict__ tokens, uint8_t *__restrict__ accept,
                                            int32_t *__restrict__ status, int N, int log2v, uint64_t limit,
                                            int rule, float conf_eps, uint64_t seed, uint32_t canvas_id,
                                            uint32_t step, int mask_id, int32_t *host_status,
                                            const float2 *__restrict__ pred, int32_t *__restrict__ pred_prev,
                                            int stable_rule) {
  __shared__ __align__(16) uint64_t keys[256];
  __shared__ uint64_t fix[4];
  __shared__ int acc_s[256];
  __shared__ float fmin_s[4], fmax_s[4], fsum_s[4];
  const int i = threadIdx.x;

  float h = 0.f;
  int32_t old = 0, p = 0, p_prev = 0, cand = 0;
  if (i < N) {  // every load up front, so their latencies overlap
    h = entropy[i];
    if (h <= 0.f) h = 0.f;  // clamp; NaN passes through
    old = tokens[i];
    cand = argmax[i];
    p = __float_as_int(pred[i].x);
    p_prev = pred_prev[i];
  }
  // masked sampler: a decided (locked) position takes no part in the walk;
  // its key sorts after every walked one and it adds nothing to their sums
  const bool walked = i < N && (mask_id < 0 || old == mask_id);
  const uint64_t key = walked ? (((uint64_t)__float_as_uint(h) << 32) | (uint32_t)i) : ~0ull;
  // h >= +0 or NaN, so the float bits order the finite entropies; NaN, inf
  // and absurd values sort after every finite one and end the walk
  acc_s[i] = 0;

  // Bitonic sort of the 256 keys, ascending, thread t ending with the key of
  // rank t: exchanges at distances below 64 go through the wavefront's lane
  // shuffles, the distances 64 and 128 through LDS.
  uint64_t k = key;
  for (int size = 2; size <= 256; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      uint64_t other;
      if (stride >= 64) {
        __syncthreads();  // the previous exchange's reads are done
        keys[i] = k;
        __syncthreads();
        other = keys[i ^ stride];
      } else {
        other = shfl_xor_u64(k, stride);
      }
      // a lower-index element keeps the smaller key in an ascending run
      const bool keep_min = ((i & stride) == 0) == ((i & size) == 0);
      k = keep_min ? (k < other ? k : other) : (k < other ? other : k);
    }
  }
  // rank t's fixed-point entropy and the inclusive prefix sum over ranks
  // (64-bit integers: exact, the same in any order)
  const float hr = __uint_as_float((uint32_t)(k >> 32));
  const bool finite_r = k != ~0ull && hr < 1048576.0f;
  const uint64_t qr = finite_r ? (uint64_t)((double)hr * 4294967296.0) : 0ull;
  uint64_t incl = qr;
  const int lane = i & 63, wave = i >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t v = shfl_up_u64(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) fix[wave] = incl;  // the wavefront's total
  __syncthreads();
  for (int w = 0; w < wave; ++w) incl += fix[w];
  // below = the entropies ranked before this one; with SUM_MINUS_MAX the
  // test drops the current (largest so far) term.  The tests grow with the
  // rank, so accepting every rank whose test holds is the sequential walk.
  const uint64_t below = incl - qr;
  const uint64_t test = (rule == DG_ACCEPT_CUMSUM) ? incl : below;
  if (finite_r && test <= limit) acc_s[(uint32_t)k] = 1;  // finite keys carry their position
  __syncthreads();
  const int acc_here = acc_s[i];

  // re-noise, new canvas, flags
  int changed = 0, conf = 1, acc = 0, isnan_ = 0, pchanged = 0;
  float hmin = INFINITY, hmax = -INFINITY, hsum = 0.f;
  int masked = 0;
  if (i < N) {
    // [P3] §5.3 / [P5]: is this position's prediction the previous step's?
    // (no previous step at step 0; a NaN entropy has no prediction to compare)
    pchanged = step == 0u || p != p_prev || h != h;
    pred_prev[i] = p;
    acc = acc_here;
    const int32_t t = acc ? cand
                          : (mask_id >= 0 ? old : uniform_token(seed, (uint32_t)i, step, canvas_id, 1u, log2v));
    tokens[i] = t;
    masked = mask_id >= 0 && t == mask_id;
    accept[i] = (uint8_t)acc;
    changed = (t != old);
    conf = (h < conf_eps);  // false for NaN
    isnan_ = (h != h);
    hmin = fminf(hmin, h);
    hmax = fmaxf(hmax, h);
    hsum = isnan_ ? 0.f : h;
  }
  const int any_changed = __syncthreads_or(changed);
  const int any_pchanged = __syncthreads_or(pchanged);
  const int all_conf = __syncthreads_and(conf);
  const int n_acc = __syncthreads_count(acc);
  const int n_nan = __syncthreads_count(isnan_);
  const int n_masked = __syncthreads_count(masked);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    hmin = fminf(hmin, __shfl_xor(hmin, o));
    hmax = fmaxf(hmax, __shfl_xor(hmax, o));
    hsum += __shfl_xor(hsum, o);
  }
  if ((i & 63) == 0) {
    fmin_s[i >> 6] = hmin;
    fmax_s[i >> 6] = hmax;
    fsum_s[i >> 6] = hsum;
  }
  __syncthreads();
  if (i == 0) {
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      fmin_s[0] = fminf(fmin_s[0], fmin_s[w]);
      fmax_s[0] = fmaxf(fmax_s[0], fmax_s[w]);
      fsum_s[0] += fsum_s[w];
    }
    const int stable_old = status[DG_ST_STABLE];
    status[DG_ST_ALLCONF] = all_conf;
    status[DG_ST_CHANGED] = any_changed;
    status[DG_ST_PRED_CHANGED] = any_pchanged;
    status[DG_ST_STABLE] = (stable_rule == DG_STABLE_CANVAS ? any_changed : any_pchanged) ? 0 : stable_old + 1;
    status[DG_ST_ACCEPTED] = n_acc;
    status[DG_ST_NAN] = n_nan;
    status[DG_ST_STEP] = (int32_t)step;
    status[DG_ST_HMIN] = __float_as_int(fmin_s[0]);
    status[DG_ST_HMAX] = __float_as_int(fmax_s[0]);
    status[DG_ST_HMEAN] = __float_as_int(N > n_nan ? fsum_s[0] / (float)(N - n_nan) : 0.f);
    status[DG_ST_MASKED] = mask_id >= 0 ? n_masked : -1;
    if (host_status) {  // the host's copy: every other word first, the step word last
      for (int w = 0; w < DG_STATUS_WORDS; ++w)
        if (w != DG_ST_STEP) host_status[w] = status[w];
      __threadfence_system();
      host_status[DG_ST_STEP] = (int32_t)step;
      __threadfence_system();
    }
  }
}

// One workgroup per canvas (a single canvas is a batch of one).
__global__ void __launch_bounds__(256) select_batch_kernel(SelectBatch bt, int N, int log2v, uint64_t limit,
                                                           int rule, float conf_eps, int mask_id, int stable_rule) {
  const int c = blockIdx.x;
  select_body(bt.entropy[c], bt.argmax[c], bt.tokens[c], bt.accept[c], bt.status[c], N, log2v, limit, rule,
              conf_eps, bt.seed[c], bt.canvas_id[c], bt.step[c], mask_id, bt.host_status[c], bt.pred[c],
              bt.pred_prev[c], stable_rule);
}

// gamma (nats) -> the 2^-32-nat fixed-point limit, saturating
static uint64_t select_limit(double gamma) {
  uint64_t limit = 0;
  if (gamma > 0.0) {
    const double x = gamma * 4294967296.0;
    limit = (x >= 18446744073709551615.0) ? ~0ull : (uint64_t)x;
  }
  return limit;
}

hipError_t select_step_batch(const SelectBatch &bt, int B, int N, int log2v, double gamma, int rule,
                             float conf_eps, int mask_id, int stable_rule, hipStream_t s) {
  if (B < 1 || B > ES_MAX_BATCH || N < 1 || N > 256) return hipErrorInvalidValue;
  for (int c = 0; c < B; ++c)
    if (!bt.pred[c] || !bt.pred_prev[c]) return hipErrorInvalidValue;
  hipLaunchKernelGGL(select_batch_kernel, dim3(B), dim3(256), 0, s, bt, N, log2v, select_limit(gamma), rule,
                     conf_eps, mask_id, stable_rule);
  return hipGetLastError();
}

__global__ void philox_test_kernel(const uint32_t *ctr, uint32_t k0, uint32_t k1, uint32_t *out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const Philox4 o = philox4x32_10(ctr[4 * i], ctr[4 * i + 1], ctr[4 * i + 2], ctr[4 * i + 3], k0, k1);
  for (int k = 0; k < 4; ++k) out[4 * i + k] = o.v[k];
}

hipError_t philox_test(const uint32_t *ctr, uint32_t k0, uint32_t k1, uint32_t *out, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(philox_test_kernel, dim3((n + 255) / 256), dim3(256), 0, s, ctr, k0, k1, out, n);
  return hipGetLastError();
}

}  // namespace dg
